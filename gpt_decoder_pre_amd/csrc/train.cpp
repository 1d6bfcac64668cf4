// Training-loop runtime around the step: learning-rate schedule and the
// sequential loader over memory-mapped token shards (gpt2_train.h).
#include "gpt2_train.h"

#include <fcntl.h>
#include <hip/hip_runtime.h>
#include <sys/mman.h>
#include <sys/stat.h>
#include <unistd.h>

#include <cmath>
#include <cstring>
#include <string>
#include <vector>

extern "C" double gpt2_lr_at(const gpt2_lr_schedule* s, int64_t step) {
  if (!s || s->warmup_steps < 1 || s->max_steps <= s->warmup_steps || step < 0) return NAN;
  if (step < s->warmup_steps) return s->max_lr * (double)(step + 1) / (double)s->warmup_steps;
  if (step > s->max_steps) return s->min_lr;
  const double r = (double)(step - s->warmup_steps) / (double)(s->max_steps - s->warmup_steps);
  return s->min_lr + 0.5 * (1.0 + std::cos(M_PI * r)) * (s->max_lr - s->min_lr);
}

namespace {

struct Shard {
  std::string path;
  const uint8_t* map = nullptr;
  size_t bytes = 0;
  int64_t n = 0;  // ids
};

}  // namespace

struct gpt2_loader {
  std::vector<Shard> shards;
  int32_t dtype = 0, vocab = 0;
  int k = 0, B = 0, T = 0;
  int64_t window = 0;  // k B T + 1
  int64_t shard = 0, pos = 0;
  // two pinned staging buffers of 2 (k B T) ids; a buffer is refilled only
  // after the copy that last read it has completed (its event)
  int32_t* stage[2] = {nullptr, nullptr};
  hipEvent_t done[2] = {nullptr, nullptr};
  bool pending[2] = {false, false};
  int next_slot = 0;
};

namespace {

bool fits(const gpt2_loader* ld, int64_t shard, int64_t pos) {
  return shard >= 0 && shard < (int64_t)ld->shards.size() && pos >= 0 &&
         pos + ld->window <= ld->shards[shard].n;
}

// The next shard (cyclically) holding one whole window, starting at `from`.
int64_t usable_from(const gpt2_loader* ld, int64_t from) {
  const int64_t ns = (int64_t)ld->shards.size();
  for (int64_t d = 0; d < ns; ++d) {
    const int64_t s = (from + d) % ns;
    if (ld->shards[s].n >= ld->window) return s;
  }
  return -1;
}

// Fills x and y (k B T each) from the current window; checks the ids.
int fill(const gpt2_loader* ld, int32_t* x, int32_t* y) {
  const Shard& s = ld->shards[ld->shard];
  const int64_t n = ld->window - 1;
  const uint8_t* base = s.map + (ld->dtype == 0 ? 2 : 4) * ld->pos;
  bool bad = false;
  if (ld->dtype == 0) {
    const uint16_t* w = reinterpret_cast<const uint16_t*>(base);
    for (int64_t i = 0; i <= n; ++i) {
      const int32_t v = (int32_t)w[i];
      bad |= v >= ld->vocab;
      if (i < n) x[i] = v;
      if (i > 0) y[i - 1] = v;
    }
  } else {
    for (int64_t i = 0; i <= n; ++i) {
      int32_t v;
      memcpy(&v, base + 4 * i, 4);
      bad |= v < 0 || v >= ld->vocab;
      if (i < n) x[i] = v;
      if (i > 0) y[i - 1] = v;
    }
  }
  return bad ? GPT2_ERR_TOKEN : GPT2_OK;
}

void advance(gpt2_loader* ld) {
  ld->pos += ld->window - 1;
  if (!fits(ld, ld->shard, ld->pos)) {
    ld->shard = usable_from(ld, ld->shard + 1);
    ld->pos = 0;
  }
  // ask the kernel to start reading the following window's pages
  const Shard& s = ld->shards[ld->shard];
  const size_t esz = ld->dtype == 0 ? 2 : 4;
  const size_t page = 4096;
  const size_t lo = (size_t)ld->pos * esz / page * page;
  const size_t hi = std::min(s.bytes, (size_t)(ld->pos + ld->window) * esz);
  if (hi > lo) (void)madvise(const_cast<uint8_t*>(s.map) + lo, hi - lo, MADV_WILLNEED);
}

void unmap_all(gpt2_loader* ld) {
  for (Shard& s : ld->shards)
    if (s.map) munmap(const_cast<uint8_t*>(s.map), s.bytes);
  ld->shards.clear();
}

}  // namespace

extern "C" {

int gpt2_loader_open(const char* const* paths, int n_shards, int32_t dtype, int32_t vocab_size, int k, int B, int T,
                     gpt2_loader** out) {
  if (!paths || !out || n_shards < 1 || k < 1 || B < 1 || T < 1 || vocab_size < 1 || (dtype != 0 && dtype != 1))
    return GPT2_ERR_ARG;
  if ((int64_t)k * B * T > ((int64_t)1 << 31)) return GPT2_ERR_ARG;
  gpt2_loader* ld = new gpt2_loader();
  ld->dtype = dtype;
  ld->vocab = vocab_size;
  ld->k = k;
  ld->B = B;
  ld->T = T;
  ld->window = (int64_t)k * B * T + 1;
  const size_t esz = dtype == 0 ? 2 : 4;
  for (int i = 0; i < n_shards; ++i) {
    Shard s;
    if (!paths[i]) {
      unmap_all(ld);
      delete ld;
      return GPT2_ERR_ARG;
    }
    s.path = paths[i];
    const int fd = open(paths[i], O_RDONLY);
    struct stat st;
    if (fd < 0 || fstat(fd, &st) != 0 || st.st_size % esz != 0) {
      if (fd >= 0) close(fd);
      unmap_all(ld);
      delete ld;
      return GPT2_ERR_IO;
    }
    s.bytes = (size_t)st.st_size;
    s.n = (int64_t)(s.bytes / esz);
    if (s.bytes > 0) {
      void* m = mmap(nullptr, s.bytes, PROT_READ, MAP_PRIVATE, fd, 0);
      if (m == MAP_FAILED) {
        close(fd);
        unmap_all(ld);
        delete ld;
        return GPT2_ERR_IO;
      }
      s.map = static_cast<const uint8_t*>(m);
    }
    close(fd);
    ld->shards.push_back(s);
  }
  ld->shard = usable_from(ld, 0);
  if (ld->shard < 0) {  // the data is too small for one batch
    unmap_all(ld);
    delete ld;
    return GPT2_ERR_BATCH;
  }
  ld->pos = 0;
  *out = ld;
  return GPT2_OK;
}

int gpt2_loader_next_host(gpt2_loader* ld, int32_t* h_idx, int32_t* h_targets) {
  if (!ld || !h_idx || !h_targets) return GPT2_ERR_ARG;
  const int e = fill(ld, h_idx, h_targets);
  if (e != GPT2_OK) return e;
  advance(ld);
  return GPT2_OK;
}

int gpt2_loader_next(gpt2_loader* ld, int32_t* d_idx, int32_t* d_targets, void* hip_stream) {
  if (!ld || !d_idx || !d_targets) return GPT2_ERR_ARG;
  const int64_t n = ld->window - 1;
  const int slot = ld->next_slot;
  if (!ld->stage[slot]) {
    if (hipHostMalloc((void**)&ld->stage[slot], 2 * n * sizeof(int32_t), hipHostMallocDefault) != hipSuccess ||
        hipEventCreateWithFlags(&ld->done[slot], hipEventDisableTiming) != hipSuccess)
      return GPT2_ERR_HIP;
  }
  if (ld->pending[slot]) {  // the copy that last read this buffer must be complete
    if (hipEventSynchronize(ld->done[slot]) != hipSuccess) return GPT2_ERR_HIP;
    ld->pending[slot] = false;
  }
  int32_t* x = ld->stage[slot];
  int32_t* y = x + n;
  const int e = fill(ld, x, y);
  if (e != GPT2_OK) return e;
  hipStream_t s = (hipStream_t)hip_stream;
  if (hipMemcpyAsync(d_idx, x, n * sizeof(int32_t), hipMemcpyHostToDevice, s) != hipSuccess ||
      hipMemcpyAsync(d_targets, y, n * sizeof(int32_t), hipMemcpyHostToDevice, s) != hipSuccess ||
      hipEventRecord(ld->done[slot], s) != hipSuccess)
    return GPT2_ERR_HIP;
  ld->pending[slot] = true;
  ld->next_slot ^= 1;
  advance(ld);
  return GPT2_OK;
}

int gpt2_loader_state(const gpt2_loader* ld, int64_t* shard, int64_t* pos) {
  if (!ld || !shard || !pos) return GPT2_ERR_ARG;
  *shard = ld->shard;
  *pos = ld->pos;
  return GPT2_OK;
}

int gpt2_loader_seek(gpt2_loader* ld, int64_t shard, int64_t pos) {
  if (!ld || !fits(ld, shard, pos)) return GPT2_ERR_ARG;
  ld->shard = shard;
  ld->pos = pos;
  return GPT2_OK;
}

void gpt2_loader_close(gpt2_loader* ld) {
  if (!ld) return;
  for (int i = 0; i < 2; ++i) {
    if (ld->pending[i]) (void)hipEventSynchronize(ld->done[i]);
    if (ld->done[i]) (void)hipEventDestroy(ld->done[i]);
    if (ld->stage[i]) (void)hipHostFree(ld->stage[i]);
  }
  unmap_all(ld);
  delete ld;
}

}  // extern "C"
