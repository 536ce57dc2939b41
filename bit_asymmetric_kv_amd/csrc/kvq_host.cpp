// Host side of the C ABI: argument validation, memory layout, the host mirror of
// per-sequence lengths, the residual-window bookkeeping, and kernel launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/kvq.h"
#include "kvq_internal.h"

using kvq::Layout;
using kvq::SeqDesc;

namespace {

thread_local char g_err[512] = "";

kvq_status fail(kvq_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

kvq_status ok() {
  g_err[0] = '\0';
  return KVQ_OK;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Quantized-token count of the residual rule: G * floor(max(0, T - o - R) / G), o = 1
// with an attention sink (its groups start at token 1).
int64_t quantized_count(int64_t T, int64_t R, int sink) {
  int64_t over = T - sink - R;
  if (over <= 0) return 0;
  return (over / kvq::kGroup) * kvq::kGroup;
}

Layout make_layout(const kvq_config* cfg);

kvq_status validate(const kvq_config* cfg) {
  if (!cfg) return fail(KVQ_ERR_INVALID_ARG, "config is NULL");
  if (cfg->batch < 1) return fail(KVQ_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", cfg->batch);
  if (cfg->num_kv_heads < 1) return fail(KVQ_ERR_INVALID_ARG, "num_kv_heads must be >= 1");
  if (cfg->num_q_heads < 1 || cfg->num_q_heads % cfg->num_kv_heads)
    return fail(KVQ_ERR_INVALID_ARG, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                cfg->num_q_heads, cfg->num_kv_heads);
  int ratio = cfg->num_q_heads / cfg->num_kv_heads;
  if (ratio != 1 && ratio != 2 && ratio != 4 && ratio != 8)
    return fail(KVQ_ERR_INVALID_ARG, "num_q_heads / num_kv_heads must be 1, 2, 4 or 8 (got %d)", ratio);
  if (cfg->head_dim != kvq::kHeadDim)
    return fail(KVQ_ERR_INVALID_ARG, "head_dim must be 128 (got %d)", cfg->head_dim);
  if (cfg->bits < 2 || cfg->bits > 4)
    return fail(KVQ_ERR_INVALID_ARG, "bits must be 2, 3 or 4 (got %d)", cfg->bits);
  if (cfg->group != kvq::kGroup)
    return fail(KVQ_ERR_INVALID_ARG, "group must be 32 (got %d)", cfg->group);
  if (cfg->head_dim % cfg->group)
    return fail(KVQ_ERR_INVALID_ARG, "head_dim must be a multiple of group");
  if (cfg->residual < 0 || cfg->residual % cfg->group || cfg->residual > kvq::kMaxResidual)
    return fail(KVQ_ERR_INVALID_ARG, "residual must be a multiple of group in [0, 4096] (got %d)",
                cfg->residual);
  if (cfg->rotate != 0 && cfg->rotate != 1) return fail(KVQ_ERR_INVALID_ARG, "rotate must be 0 or 1");
  if (cfg->max_tokens < 1 || cfg->max_tokens > (int64_t(1) << 30))
    return fail(KVQ_ERR_INVALID_ARG, "max_tokens must be in [1, 2^30]");
  if (cfg->sink != 0 && cfg->sink != 1) return fail(KVQ_ERR_INVALID_ARG, "sink must be 0 or 1");
  if (cfg->rope != 0 && cfg->rope != 1) return fail(KVQ_ERR_INVALID_ARG, "rope must be 0 or 1");
  if (cfg->rope && cfg->rotate)
    return fail(KVQ_ERR_INVALID_ARG, "pre-RoPE keys and the Walsh-Hadamard rotation cannot be combined");
  if (!(cfg->rope_base >= 0.0f) || std::isinf(cfg->rope_base) || (cfg->rope_base > 0.0f && cfg->rope_base <= 1.0f))
    return fail(KVQ_ERR_INVALID_ARG, "rope_base must be 0 (10000) or a finite value above 1");
  if (!(cfg->softmax_scale >= 0.0f) || std::isinf(cfg->softmax_scale))
    return fail(KVQ_ERR_INVALID_ARG, "softmax_scale must be finite and >= 0");
  if (cfg->page_groups < 0 || cfg->page_groups > kvq::kMaxPageGroups ||
      (cfg->page_groups & (cfg->page_groups - 1)))
    return fail(KVQ_ERR_INVALID_ARG, "page_groups must be 0 or a power of two up to %d", kvq::kMaxPageGroups);
  if (cfg->page_groups > 0 && (cfg->pool_pages < 1 || cfg->pool_pages > INT32_MAX))
    return fail(KVQ_ERR_INVALID_ARG, "pool_pages must be in [1, 2^31 - 1] for a paged cache");
  // Launch grids: the append kernels put the sequence in grid.z and the kv-head in
  // grid.y, the combine kernel the sequence in grid.y (at most 65535 each); the
  // decode kernel's 1-D grid holds (splits + window workgroups) per (sequence,
  // kv-head), at most 2^31 - 1 workgroups.
  if (cfg->batch > kvq::kMaxGridYZ || cfg->num_kv_heads > kvq::kMaxGridYZ)
    return fail(KVQ_ERR_INVALID_ARG, "batch (%d) and num_kv_heads (%d) must be at most %d (launch grid limit)",
                cfg->batch, cfg->num_kv_heads, kvq::kMaxGridYZ);
  const Layout L = make_layout(cfg);
  if (int64_t(L.B) * L.Hkv * (L.max_splits + L.win_blocks) > INT32_MAX)
    return fail(KVQ_ERR_INVALID_ARG,
                "batch * num_kv_heads * (%d splits + %d window workgroups) exceeds the 2^31 - 1 workgroups of "
                "a launch", L.max_splits, L.win_blocks);
  return ok();
}

Layout make_layout(const kvq_config* cfg) {
  Layout L{};
  L.B = cfg->batch;
  L.Hq = cfg->num_q_heads;
  L.Hkv = cfg->num_kv_heads;
  L.bits = cfg->bits;
  L.R = cfg->residual;
  L.W = cfg->residual + kvq::kGroup;
  L.sink = cfg->sink;
  L.RS = L.W + L.sink;
  L.rope = cfg->rope;
  L.gcap = (cfg->max_tokens + kvq::kGroup - 1) / kvq::kGroup;
  L.group_bytes = kvq_group_bytes(cfg->bits);
  int64_t ms = (L.gcap + kvq::kMinGroupsPerSplit - 1) / kvq::kMinGroupsPerSplit;
  L.max_splits = int32_t(std::max<int64_t>(1, std::min<int64_t>(ms, kvq::kMaxSplits)));
  const int32_t win_chunks = L.R / kvq::kGroup + 1 + L.sink;  // window < R + G tokens, plus the sink
  L.win_blocks = (win_chunks + kvq::kWindowChunksPerBlock - 1) / kvq::kWindowChunksPerBlock;
  L.P = cfg->page_groups;
  L.max_pages = L.P ? int32_t((L.gcap + L.P - 1) / L.P) : 0;
  L.pool_pages = L.P ? cfg->pool_pages : 0;
  size_t off = 0;
  L.seq_off = off;
  off = align256(off + sizeof(SeqDesc) * size_t(L.B));
  L.table_off = off;
  off = align256(off + sizeof(int32_t) * size_t(L.B) * size_t(L.max_pages));
  L.blocks_off = off;
  if (L.P)  // the page pool: [pool_pages][Hkv][P][GB]
    off = align256(off + size_t(L.pool_pages) * L.Hkv * size_t(L.P) * L.group_bytes);
  else
    off = align256(off + size_t(L.B) * L.Hkv * size_t(L.gcap) * L.group_bytes);
  size_t ring = size_t(L.B) * L.Hkv * L.RS * kvq::kHeadDim * 2;
  L.ringk_off = off;
  off = align256(off + ring);
  L.ringv_off = off;
  off = align256(off + ring);
  L.part_off = off;
  off = align256(off + size_t(L.B) * L.Hq * size_t(L.max_splits + L.win_blocks) * kvq::kPartialStride * 4);
  // rotary tables: one row per group start position, enough for every window chunk too
  L.rope_entries = L.rope ? int32_t(L.gcap + 4) : 0;
  L.rope_off = off;
  off = align256(off + size_t(L.rope_entries) * kvq::kHeadDim * 4);
  L.ropein_off = off;
  off = align256(off + (L.rope ? size_t(kvq::kGroup) * kvq::kHeadDim * 4 : 0));
  L.total = off;
  return L;
}

constexpr int kStaging = 8;  // pinned upload buffers in flight per cache

}  // namespace

struct kvq_cache {
  kvq_config cfg;
  Layout L;
  uint8_t* base = nullptr;
  bool owned = false;
  int device = 0;
  hipStream_t create_stream = nullptr;
  std::vector<int64_t> T, Q;
  int32_t groups_per_split = 0;
  hipEvent_t prof_start = nullptr, prof_stop = nullptr;
  int resident_blocks = 0;  // decode split workgroups that fit on the device at once
  int blocks_per_cu = 0;
  SeqDesc* staging[kStaging] = {};
  hipEvent_t staging_done[kStaging] = {};
  int next_staging = 0;
  // Paged caches: the page table (pinned host copy of the device table), the pages
  // each sequence has, the owner of every pool page (-1: free), and the event of the
  // last table upload (the pinned copy is not rewritten before it has passed).
  int32_t* table = nullptr;
  std::vector<int32_t> npages, owner;
  hipEvent_t table_done = nullptr;
  // A launch of an append (or of the decode of a one-call step) failed: group
  // blocks, window slots and device records may be partly written, so every
  // sequence counts as undefined until kvq_reset_sequence has started it over.
  bool broken = false;
  std::vector<char> undefined;
};

extern "C" {

size_t kvq_group_bytes(int32_t bits) {
  if (bits < 2 || bits > 4) return 0;
  return size_t(2) * kvq::kGroup * kvq::kHeadDim * bits / 8 + 512 + 512;
}

const char* kvq_last_error(void) { return g_err; }

kvq_status kvq_cache_bytes(const kvq_config* cfg, size_t* bytes) {
  kvq_status s = validate(cfg);
  if (s != KVQ_OK) return s;
  if (!bytes) return fail(KVQ_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = make_layout(cfg).total;
  return ok();
}

void kvq_destroy(kvq_cache* c) {
  if (!c) return;
  // Best-effort teardown: there is no status to return, so a failing call does not
  // stop the release of what remains.
  (void)hipSetDevice(c->device);
  (void)hipStreamSynchronize(c->create_stream);
  for (int i = 0; i < kStaging; i++) {
    if (c->staging_done[i]) {
      (void)hipEventSynchronize(c->staging_done[i]);
      (void)hipEventDestroy(c->staging_done[i]);
    }
    if (c->staging[i]) (void)hipHostFree(c->staging[i]);
  }
  if (c->table_done) {
    (void)hipEventSynchronize(c->table_done);
    (void)hipEventDestroy(c->table_done);
  }
  if (c->table) (void)hipHostFree(c->table);
  if (c->owned && c->base) (void)hipFree(c->base);
  delete c;
}

kvq_status kvq_create(const kvq_config* cfg, void* dev_mem, size_t dev_bytes, hipStream_t stream,
                      kvq_cache** out) {
  kvq_status s = validate(cfg);
  if (s != KVQ_OK) return s;
  if (!out) return fail(KVQ_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  Layout L = make_layout(cfg);
  if (dev_mem && dev_bytes < L.total)
    return fail(KVQ_ERR_OOM, "dev_bytes %zu < required %zu", dev_bytes, L.total);
  if (dev_mem && (reinterpret_cast<uintptr_t>(dev_mem) & 255))
    return fail(KVQ_ERR_INVALID_ARG, "dev_mem must be 256-byte aligned");
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
    (void)hipGetLastError();
    return fail(KVQ_ERR_NO_DEVICE, "no HIP device available");
  }
  kvq_cache* c = new (std::nothrow) kvq_cache();
  if (!c) return fail(KVQ_ERR_OOM, "host allocation failed");
  c->cfg = *cfg;
  if (c->cfg.softmax_scale == 0.0f) c->cfg.softmax_scale = 1.0f / std::sqrt(float(cfg->head_dim));
  c->L = L;
  c->create_stream = stream;
  c->T.assign(cfg->batch, 0);
  c->Q.assign(cfg->batch, 0);
  if (hipGetDevice(&c->device) != hipSuccess) {
    (void)hipGetLastError();
    delete c;
    return fail(KVQ_ERR_NO_DEVICE, "no current HIP device");
  }
  if (dev_mem) {
    c->base = static_cast<uint8_t*>(dev_mem);
  } else {
    if (hipMalloc(reinterpret_cast<void**>(&c->base), L.total) != hipSuccess) {
      (void)hipGetLastError();
      delete c;
      return fail(KVQ_ERR_OOM, "hipMalloc of %zu bytes failed", L.total);
    }
    c->owned = true;
  }
  for (int i = 0; i < kStaging; i++) {
    if (hipHostMalloc(reinterpret_cast<void**>(&c->staging[i]), sizeof(SeqDesc) * cfg->batch) !=
            hipSuccess ||
        hipEventCreateWithFlags(&c->staging_done[i], hipEventDisableTiming) != hipSuccess) {
      (void)hipGetLastError();
      kvq_destroy(c);
      return fail(KVQ_ERR_HIP, "pinned staging allocation failed");
    }
  }
  if (hipMemsetAsync(c->base + L.seq_off, 0, sizeof(SeqDesc) * cfg->batch, stream) != hipSuccess) {
    kvq_destroy(c);
    return fail(KVQ_ERR_HIP, "clearing sequence state failed: %s", hipGetErrorString(hipGetLastError()));
  }
  if (L.P) {
    const size_t tb = sizeof(int32_t) * size_t(L.B) * size_t(L.max_pages);
    if (hipHostMalloc(reinterpret_cast<void**>(&c->table), tb) != hipSuccess ||
        hipEventCreateWithFlags(&c->table_done, hipEventDisableTiming) != hipSuccess) {
      (void)hipGetLastError();
      kvq_destroy(c);
      return fail(KVQ_ERR_HIP, "pinned page-table allocation failed");
    }
    std::fill(c->table, c->table + size_t(L.B) * L.max_pages, 0);
    c->npages.assign(cfg->batch, 0);
    c->owner.assign(size_t(L.pool_pages), -1);
    // unassigned entries point at page 0, which always exists
    if (hipMemsetAsync(c->base + L.table_off, 0, tb, stream) != hipSuccess) {
      kvq_destroy(c);
      return fail(KVQ_ERR_HIP, "clearing the page table failed: %s", hipGetErrorString(hipGetLastError()));
    }
  }
  if (L.rope) {
    const double rb = cfg->rope_base > 0.0f ? double(cfg->rope_base) : 10000.0;
    const hipError_t e = kvq::launch_rope_tables(L, c->base, rb, stream);
    if (e != hipSuccess) {
      kvq_destroy(c);
      return fail(KVQ_ERR_HIP, "building the rotary tables failed: %s", hipGetErrorString(e));
    }
  }
  *out = c;
  return ok();
}

kvq_status kvq_seq_len(const kvq_cache* c, int32_t b, int64_t* T, int64_t* Q) {
  if (!c) return fail(KVQ_ERR_INVALID_ARG, "cache is NULL");
  if (b < 0 || b >= c->cfg.batch) return fail(KVQ_ERR_INVALID_ARG, "sequence index %d out of range", b);
  if (T) *T = c->T[b];
  if (Q) *Q = c->Q[b];
  return ok();
}

kvq_status kvq_set_decode_split(kvq_cache* c, int32_t groups_per_split) {
  if (!c) return fail(KVQ_ERR_INVALID_ARG, "cache is NULL");
  if (groups_per_split != 0 &&
      (groups_per_split < kvq::kMinGroupsPerSplit || groups_per_split > (1 << 20)))
    return fail(KVQ_ERR_INVALID_ARG, "groups_per_split must be 0 or in [%d, 2^20]",
                kvq::kMinGroupsPerSplit);
  c->groups_per_split = groups_per_split;
  return ok();
}

kvq_status kvq_set_profile_events(kvq_cache* c, hipEvent_t start, hipEvent_t stop) {
  if (!c) return fail(KVQ_ERR_INVALID_ARG, "cache is NULL");
  if ((start == nullptr) != (stop == nullptr))
    return fail(KVQ_ERR_INVALID_ARG, "start and stop must both be set or both be NULL");
  c->prof_start = start;
  c->prof_stop = stop;
  return ok();
}

}  // extern "C"

namespace {

// After a failed append launch every call that reads or extends the cache is
// refused until each sequence has been reset.
kvq_status refuse_if_broken(const kvq_cache* c) {
  if (c->broken)
    return fail(KVQ_ERR_HIP,
                "an earlier append launch failed and left the cache contents undefined; reset every sequence "
                "(kvq_reset_sequence) or destroy the cache");
  return KVQ_OK;
}

kvq_status mark_broken(kvq_cache* c, kvq_status st) {
  c->broken = true;
  c->undefined.assign(c->cfg.batch, 1);
  return st;
}

// An append that has been checked and described but not yet launched.
struct PendingAppend {
  kvq::SeqArgs sa;
  std::vector<int64_t> T2, Q2;  // lengths after the append
  int32_t max_flush = 0;        // groups leaving the window, most of any sequence
  int32_t max_ring = 0;         // appended tokens staying in the window, most of any sequence
  int64_t total_new = 0;
};

// Checks an append and fills its per-sequence records (inline for small batches,
// otherwise uploaded on `stream` from pinned staging into the device state).
kvq_status prepare_append(kvq_cache* c, const void* k, const void* v, const int32_t* n_tokens, int32_t n_max,
                          hipStream_t stream, PendingAppend& pa) {
  const int B = c->cfg.batch;
  if (n_max < 0) return fail(KVQ_ERR_INVALID_ARG, "n_max must be >= 0");
  pa.total_new = 0;
  for (int b = 0; b < B; b++) {
    int64_t n = n_tokens ? n_tokens[b] : n_max;
    if (n < 0 || n > n_max)
      return fail(KVQ_ERR_INVALID_ARG, "n_tokens[%d] = %lld outside [0, n_max=%d]", b, (long long)n, n_max);
    if (c->T[b] + n > c->cfg.max_tokens)
      return fail(KVQ_ERR_CAPACITY, "sequence %d would hold %lld tokens > max_tokens %lld", b,
                  (long long)(c->T[b] + n), (long long)c->cfg.max_tokens);
    if (c->L.P) {
      const int64_t groups = quantized_count(c->T[b] + n, c->cfg.residual, c->cfg.sink) / kvq::kGroup;
      const int64_t need = (groups + c->L.P - 1) / c->L.P;
      if (need > c->npages[b])
        return fail(KVQ_ERR_CAPACITY, "sequence %d needs %lld pages for its groups and has %d", b,
                    (long long)need, c->npages[b]);
    }
    pa.total_new += n;
  }
  pa.T2 = c->T;
  pa.Q2 = c->Q;
  if (pa.total_new == 0) return ok();
  if (!k || !v) return fail(KVQ_ERR_INVALID_ARG, "k and v must be device pointers when tokens are appended");

  // Host bookkeeping: new lengths, groups leaving the window, tokens entering it.
  const bool inl = B <= kvq::kInlineSeqs;
  SeqDesc* d = pa.sa.inl;
  int slot = -1;
  if (!inl) {
    slot = c->next_staging;
    c->next_staging = (slot + 1) % kStaging;
    if (hipEventSynchronize(c->staging_done[slot]) != hipSuccess)
      return fail(KVQ_ERR_HIP, "waiting for a staging buffer failed: %s", hipGetErrorString(hipGetLastError()));
    d = c->staging[slot];
  }
  pa.max_flush = pa.max_ring = 0;
  for (int b = 0; b < B; b++) {
    int64_t n = n_tokens ? n_tokens[b] : n_max;
    pa.T2[b] = c->T[b] + n;
    pa.Q2[b] = quantized_count(pa.T2[b], c->cfg.residual, c->cfg.sink);
    d[b].t_old = int32_t(c->T[b]);
    d[b].n_new = int32_t(n);
    d[b].q_old = int32_t(c->Q[b]);
    d[b].q_new = int32_t(pa.Q2[b]);
    pa.max_flush = std::max<int32_t>(pa.max_flush, int32_t((pa.Q2[b] - c->Q[b]) / kvq::kGroup));
    // appended tokens that stay in the FP16 window (an appended sink counts as one more)
    int64_t first_kept = std::max<int64_t>(c->T[b], c->cfg.sink + pa.Q2[b]);
    const int64_t sink_new = (c->cfg.sink && c->T[b] == 0 && n > 0) ? 1 : 0;
    pa.max_ring = std::max<int32_t>(pa.max_ring,
                                    int32_t(std::max<int64_t>(0, pa.T2[b] - first_kept) + sink_new));
  }
  SeqDesc* dev_seq = reinterpret_cast<SeqDesc*>(c->base + c->L.seq_off);
  pa.sa.dev = dev_seq;
  pa.sa.state = dev_seq;
  pa.sa.inl_valid = inl ? 1 : 0;
  if (!inl && (hipMemcpyAsync(dev_seq, d, sizeof(SeqDesc) * B, hipMemcpyHostToDevice, stream) != hipSuccess ||
               hipEventRecord(c->staging_done[slot], stream) != hipSuccess))
    return fail(KVQ_ERR_HIP, "uploading sequence state failed: %s", hipGetErrorString(hipGetLastError()));
  return ok();
}

// Decode over lengths T, Q (the host mirror after any append in the same call);
// with `pa`, the decode kernel also writes that append's tokens into the window.
kvq_status launch_decode_for(kvq_cache* c, const std::vector<int64_t>& T, const std::vector<int64_t>& Q,
                             const PendingAppend* pa, const void* k, const void* v, int32_t n_max, const void* q,
                             float* out, hipStream_t stream);

}  // namespace

extern "C" {

kvq_status kvq_append(kvq_cache* c, const void* k, const void* v, const int32_t* n_tokens,
                      int32_t n_max, hipStream_t stream) {
  if (!c) return fail(KVQ_ERR_INVALID_ARG, "cache is NULL");
  if (refuse_if_broken(c) != KVQ_OK) return KVQ_ERR_HIP;
  PendingAppend pa;
  kvq_status st = prepare_append(c, k, v, n_tokens, n_max, stream, pa);
  if (st == KVQ_ERR_HIP) return mark_broken(c, st);  // the record upload may have started
  if (st != KVQ_OK || pa.total_new == 0) return st;
  hipError_t e = hipSuccess;
  if (pa.max_flush > 0)
    e = kvq::launch_flush(c->L, c->base, pa.sa, k, v, n_max, pa.max_flush, c->cfg.rotate, stream);
  // The window-write kernel always runs: with inline records it also stores them.
  if (e == hipSuccess && (pa.max_ring > 0 || pa.sa.inl_valid))
    e = kvq::launch_ring_write(c->L, c->base, pa.sa, k, v, n_max, std::max(pa.max_ring, 1), c->cfg.rotate, stream);
  if (e != hipSuccess) return mark_broken(c, fail(KVQ_ERR_HIP, "append kernels failed: %s", hipGetErrorString(e)));
  c->T = pa.T2;
  c->Q = pa.Q2;
  return ok();
}

kvq_status kvq_decode_step(kvq_cache* c, const void* k, const void* v, const int32_t* n_tokens, int32_t n_max,
                           const void* q, float* out, hipStream_t stream) {
  if (!c) return fail(KVQ_ERR_INVALID_ARG, "cache is NULL");
  if (!q || !out) return fail(KVQ_ERR_INVALID_ARG, "q and out must be device pointers");
  if (refuse_if_broken(c) != KVQ_OK) return KVQ_ERR_HIP;
  PendingAppend pa;
  // Checks that need no launch come first, so that a failing call changes nothing.
  {
    const int B = c->cfg.batch;
    if (n_max < 0) return fail(KVQ_ERR_INVALID_ARG, "n_max must be >= 0");
    for (int b = 0; b < B; b++) {
      const int64_t n = n_tokens ? n_tokens[b] : n_max;
      if (n >= 0 && n <= n_max && c->T[b] + n == 0) return fail(KVQ_ERR_EMPTY, "sequence %d holds no token", b);
    }
  }
  kvq_status st = prepare_append(c, k, v, n_tokens, n_max, stream, pa);
  if (st == KVQ_ERR_HIP) return mark_broken(c, st);  // the record upload may have started
  if (st != KVQ_OK) return st;
  // Rotated caches keep the separate window-write kernel (it rotates the new keys);
  // otherwise the decode launch writes the new window tokens itself.
  const bool fold = pa.total_new > 0 && !c->cfg.rotate;
  hipError_t e = hipSuccess;
  if (pa.total_new > 0 && pa.max_flush > 0)
    e = kvq::launch_flush(c->L, c->base, pa.sa, k, v, n_max, pa.max_flush, c->cfg.rotate, stream);
  if (e == hipSuccess && pa.total_new > 0 && !fold && (pa.max_ring > 0 || pa.sa.inl_valid))
    e = kvq::launch_ring_write(c->L, c->base, pa.sa, k, v, n_max, std::max(pa.max_ring, 1), c->cfg.rotate, stream);
  if (e != hipSuccess) return mark_broken(c, fail(KVQ_ERR_HIP, "append kernels failed: %s", hipGetErrorString(e)));
  st = launch_decode_for(c, pa.T2, pa.Q2, fold ? &pa : nullptr, k, v, n_max, q, out, stream);
  // The decode launch may already have written the appended window tokens (and,
  // with uploaded records, the device state) when it fails.
  if (st == KVQ_ERR_HIP && pa.total_new > 0) return mark_broken(c, st);
  if (st != KVQ_OK) return st;
  c->T = pa.T2;
  c->Q = pa.Q2;
  return ok();
}

kvq_status kvq_decode_attention(kvq_cache* c, const void* q, float* out, hipStream_t stream) {
  if (!c) return fail(KVQ_ERR_INVALID_ARG, "cache is NULL");
  if (!q || !out) return fail(KVQ_ERR_INVALID_ARG, "q and out must be device pointers");
  if (refuse_if_broken(c) != KVQ_OK) return KVQ_ERR_HIP;
  return launch_decode_for(c, c->T, c->Q, nullptr, nullptr, nullptr, 0, q, out, stream);
}

kvq_status kvq_read_state(kvq_cache* c, int32_t part, int32_t b, int32_t h, size_t offset,
                          void* host_dst, size_t bytes, hipStream_t stream) {
  if (!c) return fail(KVQ_ERR_INVALID_ARG, "cache is NULL");
  if (b < 0 || b >= c->cfg.batch || h < 0 || h >= c->cfg.num_kv_heads)
    return fail(KVQ_ERR_INVALID_ARG, "(b, h) = (%d, %d) out of range", b, h);
  if (!host_dst && bytes) return fail(KVQ_ERR_INVALID_ARG, "host_dst is NULL");
  const Layout& L = c->L;
  size_t region, start;
  size_t bh = size_t(b) * L.Hkv + h;
  switch (part) {
    case KVQ_PART_GROUPS:
      region = size_t(L.gcap) * L.group_bytes;
      start = L.blocks_off + bh * region;
      break;
    case KVQ_PART_RING_K:
    case KVQ_PART_RING_V:
      region = size_t(L.RS) * kvq::kHeadDim * 2;
      start = (part == KVQ_PART_RING_K ? L.ringk_off : L.ringv_off) + bh * region;
      break;
    default:
      return fail(KVQ_ERR_INVALID_ARG, "unknown part %d", part);
  }
  if (offset > region || bytes > region - offset)
    return fail(KVQ_ERR_INVALID_ARG, "range [%zu, %zu) exceeds the part's %zu bytes", offset,
                offset + bytes, region);
  if (bytes == 0) return ok();
  if (part == KVQ_PART_GROUPS && L.P) {
    // paged: gather page by page through the table
    const size_t gb = L.group_bytes;
    const kvq::GroupStore st = kvq::group_store(L, c->base);
    size_t done = 0;
    while (done < bytes) {
      const size_t pos = offset + done;
      const int64_t g = int64_t(pos / gb);
      if (g / L.P >= c->npages[b])
        return fail(KVQ_ERR_INVALID_ARG, "group %lld of sequence %d has no page", (long long)g, b);
      const size_t run = std::min(bytes - done, size_t(L.P - g % L.P) * gb - pos % gb);
      const size_t src = st.offset(b, h, g, c->table[size_t(b) * L.max_pages + g / L.P]) + pos % gb;
      if (hipMemcpyAsync(static_cast<uint8_t*>(host_dst) + done, c->base + L.blocks_off + src, run,
                         hipMemcpyDeviceToHost, stream) != hipSuccess)
        return fail(KVQ_ERR_HIP, "reading state failed: %s", hipGetErrorString(hipGetLastError()));
      done += run;
    }
    if (hipStreamSynchronize(stream) != hipSuccess)
      return fail(KVQ_ERR_HIP, "reading state failed: %s", hipGetErrorString(hipGetLastError()));
    return ok();
  }
  if (hipMemcpyAsync(host_dst, c->base + start + offset, bytes, hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return fail(KVQ_ERR_HIP, "reading state failed: %s", hipGetErrorString(hipGetLastError()));
  return ok();
}

kvq_status kvq_set_pages(kvq_cache* c, int32_t b, const int32_t* pages, int32_t n, hipStream_t stream) {
  if (!c) return fail(KVQ_ERR_INVALID_ARG, "cache is NULL");
  const Layout& L = c->L;
  if (!L.P) return fail(KVQ_ERR_INVALID_ARG, "the cache is not paged (page_groups == 0)");
  if (b < 0 || b >= c->cfg.batch) return fail(KVQ_ERR_INVALID_ARG, "sequence index %d out of range", b);
  if (n < 0 || n > L.max_pages)
    return fail(KVQ_ERR_INVALID_ARG, "n = %d outside [0, %d] pages per sequence", n, L.max_pages);
  if (n && !pages) return fail(KVQ_ERR_INVALID_ARG, "pages is NULL");
  int32_t* row = c->table + size_t(b) * L.max_pages;
  // pages holding quantized groups keep their place
  const int64_t used = (c->Q[b] / kvq::kGroup + L.P - 1) / L.P;
  if (n < used) return fail(KVQ_ERR_INVALID_ARG, "sequence %d holds groups in %lld pages; n = %d", b,
                            (long long)used, n);
  std::vector<int32_t> seen;
  seen.reserve(n);
  for (int32_t i = 0; i < n; i++) {
    const int32_t p = pages[i];
    if (p < 0 || int64_t(p) >= L.pool_pages)
      return fail(KVQ_ERR_INVALID_ARG, "page %d outside the pool of %lld", p, (long long)L.pool_pages);
    if (c->owner[p] != -1 && c->owner[p] != b)
      return fail(KVQ_ERR_INVALID_ARG, "page %d belongs to sequence %d", p, c->owner[p]);
    if (i < used && p != row[i])
      return fail(KVQ_ERR_INVALID_ARG, "page %d of sequence %d holds groups and cannot move", i, b);
    seen.push_back(p);
  }
  std::sort(seen.begin(), seen.end());
  if (std::adjacent_find(seen.begin(), seen.end()) != seen.end())
    return fail(KVQ_ERR_INVALID_ARG, "a page appears twice");
  if (hipEventSynchronize(c->table_done) != hipSuccess)
    return fail(KVQ_ERR_HIP, "waiting for the previous table upload failed");
  for (int32_t i = 0; i < c->npages[b]; i++) c->owner[row[i]] = -1;
  for (int32_t i = 0; i < n; i++) {
    row[i] = pages[i];
    c->owner[pages[i]] = b;
  }
  c->npages[b] = n;
  if (n && (hipMemcpyAsync(c->base + L.table_off + sizeof(int32_t) * size_t(b) * L.max_pages, row,
                           sizeof(int32_t) * size_t(n), hipMemcpyHostToDevice, stream) != hipSuccess ||
            hipEventRecord(c->table_done, stream) != hipSuccess))
    return fail(KVQ_ERR_HIP, "uploading the page table failed: %s", hipGetErrorString(hipGetLastError()));
  return ok();
}

kvq_status kvq_reset_sequence(kvq_cache* c, int32_t b) {
  if (!c) return fail(KVQ_ERR_INVALID_ARG, "cache is NULL");
  if (b < 0 || b >= c->cfg.batch) return fail(KVQ_ERR_INVALID_ARG, "sequence index %d out of range", b);
  c->T[b] = 0;
  c->Q[b] = 0;
  if (c->broken) {
    c->undefined[b] = 0;
    c->broken = std::find(c->undefined.begin(), c->undefined.end(), 1) != c->undefined.end();
  }
  if (c->L.P) {
    const int32_t* row = c->table + size_t(b) * c->L.max_pages;
    for (int32_t i = 0; i < c->npages[b]; i++) c->owner[row[i]] = -1;
    c->npages[b] = 0;
  }
  return ok();
}

kvq_status kvq_stream_read(const void* buf, size_t bytes, uint32_t* fold, int32_t fold_words, hipStream_t stream) {
  if (!buf || !fold) return fail(KVQ_ERR_INVALID_ARG, "buf and fold must be device pointers");
  if (bytes == 0 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return fail(KVQ_ERR_INVALID_ARG, "bytes must be a positive multiple of 16 and buf 16-byte aligned");
  if (fold_words < 1 || fold_words > kvq::kMaxStreamWorkgroups)
    return fail(KVQ_ERR_INVALID_ARG, "fold_words must be in [1, %d] (got %d)", kvq::kMaxStreamWorkgroups, fold_words);
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
    (void)hipGetLastError();
    return fail(KVQ_ERR_NO_DEVICE, "no HIP device available");
  }
  const hipError_t e = kvq::launch_stream_read(buf, bytes, fold, fold_words, stream);
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "stream read launch failed: %s", hipGetErrorString(e));
  return ok();
}

kvq_status kvq_fp16_workspace_bytes(const kvq_fp16_config* cfg, size_t* bytes) {
  if (!cfg || !bytes) return fail(KVQ_ERR_INVALID_ARG, "cfg and bytes must not be NULL");
  if (cfg->batch < 1 || cfg->num_kv_heads < 1 || cfg->num_q_heads < 1 || cfg->num_q_heads % cfg->num_kv_heads)
    return fail(KVQ_ERR_INVALID_ARG, "need batch >= 1 and num_q_heads a positive multiple of num_kv_heads");
  *bytes = size_t(cfg->batch) * cfg->num_q_heads * kvq::kFp16MaxSplits * kvq::kPartialStride * 4;
  return ok();
}

}  // extern "C"

namespace {

// Checked FP16-decode launch shape: nsplit splits of cps 32-token chunks per
// (sequence, kv-head); partials [B][Hq][nsplit][130] fp32.
struct Fp16Plan {
  int64_t nsplit = 0, cps = 0;
  float scale_log2 = 0.0f;
  size_t partial_bytes = 0;
};

// Host-side argument checks of an FP16-decode call.
kvq_status check_fp16(const kvq_fp16_config* cfg, const void* k, const void* v, const int32_t* seq_lens,
                      int64_t max_len, const void* q, const float* out) {
  if (!cfg) return fail(KVQ_ERR_INVALID_ARG, "cfg is NULL");
  const int ratio = cfg->num_kv_heads > 0 ? cfg->num_q_heads / cfg->num_kv_heads : 0;
  if (cfg->batch < 1 || cfg->num_kv_heads < 1 || cfg->num_q_heads % cfg->num_kv_heads != 0 ||
      !(ratio == 1 || ratio == 2 || ratio == 4 || ratio == 8))
    return fail(KVQ_ERR_INVALID_ARG, "batch >= 1 and num_q_heads / num_kv_heads in {1, 2, 4, 8} required");
  if (cfg->head_dim != kvq::kHeadDim) return fail(KVQ_ERR_INVALID_ARG, "head_dim must be 128");
  if (cfg->t_cap < 1 || cfg->t_cap > (int64_t(1) << 30))
    return fail(KVQ_ERR_INVALID_ARG, "t_cap must be in [1, 2^30]");
  if (max_len < 1 || max_len > cfg->t_cap)
    return fail(KVQ_ERR_INVALID_ARG, "max_len must be in [1, t_cap]");
  if (cfg->batch > kvq::kMaxGridYZ)
    return fail(KVQ_ERR_INVALID_ARG, "batch must be at most %d (launch grid limit)", kvq::kMaxGridYZ);
  if (!k || !v || !seq_lens || !q || !out)
    return fail(KVQ_ERR_INVALID_ARG, "k, v, seq_lens, q and out must be device pointers");
  return ok();
}

// The split plan of a checked FP16-decode call (queries the current device).
kvq_status plan_fp16(const kvq_fp16_config* cfg, int64_t max_len, Fp16Plan& p) {
  int ndev = 0, dev = 0, cus = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1) {
    (void)hipGetLastError();
    return fail(KVQ_ERR_NO_DEVICE, "no HIP device available");
  }
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return fail(KVQ_ERR_HIP, "device query failed: %s", hipGetErrorString(hipGetLastError()));
  // Two workgroups per compute unit (the kernel's occupancy) in one round, at least
  // one chunk per wave.
  const int64_t bh = int64_t(cfg->batch) * cfg->num_kv_heads;
  const int64_t nch = (max_len + 31) / 32;
  int64_t splits = std::max<int64_t>(1, (int64_t(cus) * 2) / bh);
  int64_t cps = std::max<int64_t>(4, (nch + splits - 1) / splits);
  int64_t nsplit = (nch + cps - 1) / cps;
  if (nsplit > kvq::kFp16MaxSplits) {
    cps = (nch + kvq::kFp16MaxSplits - 1) / kvq::kFp16MaxSplits;
    nsplit = (nch + cps - 1) / cps;
  }
  if (nsplit * bh > INT32_MAX) return fail(KVQ_ERR_INVALID_ARG, "too many workgroups for one launch");
  const float scale = cfg->softmax_scale > 0.0f ? cfg->softmax_scale : 1.0f / std::sqrt(float(cfg->head_dim));
  p.nsplit = nsplit;
  p.cps = cps;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.partial_bytes = size_t(cfg->batch) * cfg->num_q_heads * size_t(nsplit) * kvq::kPartialStride * 4;
  return ok();
}

kvq_status launch_fp16_plan(const kvq_fp16_config* cfg, const Fp16Plan& p, const void* k, const void* v,
                            const int32_t* seq_lens, const void* q, float* out, float* part, hipStream_t stream) {
  const hipError_t e = kvq::launch_fp16_decode(k, v, seq_lens, cfg->t_cap, cfg->batch, cfg->num_q_heads,
                                               cfg->num_kv_heads, p.scale_log2, q, out, part, int(p.nsplit),
                                               int(p.cps), stream);
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "fp16 decode launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace

extern "C" {

kvq_status kvq_fp16_decode_attention(const kvq_fp16_config* cfg, const void* k, const void* v,
                                     const int32_t* seq_lens, int64_t max_len, const void* q, float* out,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  kvq_status st = check_fp16(cfg, k, v, seq_lens, max_len, q, out);
  if (st != KVQ_OK) return st;
  if (!workspace) return fail(KVQ_ERR_INVALID_ARG, "workspace must be a device pointer");
  size_t need = 0;
  st = kvq_fp16_workspace_bytes(cfg, &need);
  if (st != KVQ_OK) return st;
  if (workspace_bytes < need) return fail(KVQ_ERR_OOM, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  Fp16Plan p;
  st = plan_fp16(cfg, max_len, p);
  if (st != KVQ_OK) return st;
  return launch_fp16_plan(cfg, p, k, v, seq_lens, q, out, static_cast<float*>(workspace), stream);
}

kvq_status kvq_fp16_decode_attention_noalloc(const kvq_fp16_config* cfg, const void* k, const void* v,
                                             const int32_t* seq_lens, int64_t max_len, const void* q, float* out,
                                             hipStream_t stream) {
  kvq_status st = check_fp16(cfg, k, v, seq_lens, max_len, q, out);
  if (st != KVQ_OK) return st;
  Fp16Plan p;
  st = plan_fp16(cfg, max_len, p);
  if (st != KVQ_OK) return st;
  if (p.partial_bytes > kvq::kFp16ScratchBytes)
    return fail(KVQ_ERR_CAPACITY,
                "this shape needs %zu bytes of split partials; the static scratch holds %zu (use "
                "kvq_fp16_decode_attention with a workspace)",
                p.partial_bytes, kvq::kFp16ScratchBytes);
  void* part = nullptr;
  const hipError_t e = kvq::fp16_scratch(&part);
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "looking up the static scratch failed: %s", hipGetErrorString(e));
  return launch_fp16_plan(cfg, p, k, v, seq_lens, q, out, static_cast<float*>(part), stream);
}

}  // extern "C"

namespace {

kvq_status launch_decode_for(kvq_cache* c, const std::vector<int64_t>& T, const std::vector<int64_t>& Q,
                             const PendingAppend* pa, const void* k, const void* v, int32_t n_max, const void* q,
                             float* out, hipStream_t stream) {
  const int B = c->cfg.batch, Hkv = c->cfg.num_kv_heads;
  int64_t max_groups = 0, sum_groups = 0;
  for (int b = 0; b < B; b++) {
    if (T[b] == 0) return fail(KVQ_ERR_EMPTY, "sequence %d holds no token", b);
    max_groups = std::max(max_groups, Q[b] / kvq::kGroup);
    sum_groups += Q[b] / kvq::kGroup;
  }
  // Equal lengths: one round of equal workgroups. Unequal lengths: about one and a
  // half rounds of smaller ones, longest sequences first.
  const bool uniform_lengths = sum_groups == max_groups * B;
  int64_t gps = c->groups_per_split;
  if (gps == 0 && max_groups > 0) {
    // As many split workgroups as fit on the device at once next to the FP16-window
    // workgroups, each reading about the same number of groups, so a sequence gets
    // splits in proportion to its length. With unequal lengths the splits are made
    // 1.5 times finer, so that the short sequences' single splits fill the slots the
    // long ones leave (64 sequences of 2K-32K tokens: 1.5 rounds measured 6 % faster
    // than 2 or 3 rounds, whose workgroups each pay the start-up and merge again, and
    // faster than 1.1 rounds, whose last workgroups run alone).
    if (c->resident_blocks == 0) {
      c->blocks_per_cu = kvq::decode_blocks_per_cu(c->cfg.bits, c->cfg.num_q_heads / c->cfg.num_kv_heads,
                                                   c->cfg.rope);
      c->resident_blocks = std::max(1, c->blocks_per_cu * kvq::device_compute_units());
    }
    const int64_t win = int64_t(B) * Hkv * c->L.win_blocks;
    const int64_t slots = std::max<int64_t>(int64_t(B) * Hkv,
                                            c->resident_blocks - std::min<int64_t>(win, c->resident_blocks / 4));
    const int64_t half_rounds = uniform_lengths ? 2 : 3;
    gps = std::max<int64_t>(kvq::kMinGroupsPerSplit,
                            (2 * sum_groups * Hkv + slots * half_rounds - 1) / (slots * half_rounds));
  }
  if (gps == 0) gps = kvq::kMinGroupsPerSplit;
  // Every sequence's split count must stay within the partial slots.
  gps = std::max<int64_t>(gps, (max_groups + c->L.max_splits - 1) / c->L.max_splits);
  // Equal sequences: keep the split count and spread the groups evenly over the
  // splits. Rounding the count up left the last split of every sequence short (8
  // sequences x 32 KV heads at 32K tokens: splits of 680 and 340 groups, so half the
  // workgroups ended early and the long ones finished at one wave per SIMD; even
  // splits of 510 made that step 11 % shorter).
  if (c->groups_per_split == 0 && uniform_lengths && max_groups > 0) {
    const int64_t n = (max_groups + gps - 1) / gps;
    gps = std::max<int64_t>(kvq::kMinGroupsPerSplit, (max_groups + n - 1) / n);
    gps = std::max<int64_t>(gps, (max_groups + c->L.max_splits - 1) / c->L.max_splits);
  }
  kvq::SplitPlan plan{};
  int64_t max_split = 0;
  if (B <= kvq::kInlineSeqs) {
    // Longest sequences first, so that their splits are dispatched first.
    int order[kvq::kInlineSeqs];
    for (int b = 0; b < B; b++) order[b] = b;
    std::stable_sort(order, order + B, [&](int x, int y) { return Q[x] > Q[y]; });
    plan.use_prefix = 1;
    plan.prefix[0] = 0;
    for (int p = 0; p < B; p++) {
      const int b = order[p];
      const int64_t n = (Q[b] / kvq::kGroup + gps - 1) / gps;
      max_split = std::max(max_split, n);
      plan.seq[p] = b;
      plan.count[b] = int32_t(n);
      plan.prefix[p + 1] = plan.prefix[p] + int32_t(n);
    }
  } else {
    plan.use_prefix = 0;
    max_split = (max_groups + gps - 1) / gps;
    plan.uniform = int32_t(max_split);
  }
  plan.pstride = int32_t(max_split) + c->L.win_blocks;
  // One round of equal sequences' splits at two workgroups per compute unit: the
  // dispatcher fills every compute unit's first slot before its second, and a compute
  // unit then issues from its older workgroup first, so the younger one trails and
  // ends alone. Giving the first-dispatched half of the splits 1.7 times the groups of
  // the second half lets both end together (measured against equal splits: about 7 %
  // shorter steps at 128K tokens; 1.4, 1.5, 2, 2.5 and 3 measured slower than 1.7).
  // FP16-window workgroups that do not fit in the same round follow the splits and do
  // not change their placement (8 sequences x 32 KV heads at 32K tokens: 6 % shorter
  // steps than equal splits). Explicit split sizes keep equal splits.
  plan.older_weight = 0.0f;
  if (c->groups_per_split == 0 && uniform_lengths && c->blocks_per_cu == 2 && max_split >= 2 &&
      max_split * int64_t(B) * Hkv <= c->resident_blocks)
    plan.older_weight = 1.7f;
  const float scale_log2 = c->cfg.softmax_scale * 1.4426950408889634f;
  const SeqDesc* dev_seq = reinterpret_cast<const SeqDesc*>(c->base + c->L.seq_off);
  kvq::AppendArgs app{};
  if (pa) {
    app.pending = 1;
    app.k = k;
    app.v = v;
    app.n_max = n_max;
    app.seq = pa->sa;
  } else if (B <= kvq::kInlineSeqs) {
    // no append in this launch: the records the kernels read are the host mirror's
    for (int b = 0; b < B; b++)
      app.seq.inl[b] = SeqDesc{int32_t(T[b]), 0, int32_t(Q[b]), int32_t(Q[b])};
    app.seq.inl_valid = 1;
  }
  hipError_t e = kvq::launch_decode(c->L, c->base, dev_seq, app, q, out, int32_t(gps), plan,
                                    scale_log2, c->cfg.rotate, stream, c->prof_start, c->prof_stop);
  if (e != hipSuccess) return fail(KVQ_ERR_HIP, "decode kernels failed: %s", hipGetErrorString(e));
  return ok();
}

}  // namespace
