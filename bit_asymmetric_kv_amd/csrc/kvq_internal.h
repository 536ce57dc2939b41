// Internal declarations shared by the host library and its kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvq {

constexpr int kHeadDim = 128;
constexpr int kGroup = 32;
constexpr int kPartialStride = kHeadDim + 2;  // m (log2 domain), l, o[128] per partial
constexpr int kMinGroupsPerSplit = 4;
constexpr int kMaxSplits = 2048;
constexpr int kMaxResidual = 4096;
constexpr int kMaxPageGroups = 1 << 16;  // groups per page of a paged cache
constexpr int kMaxGridYZ = 65535;        // launch grid limit in y and z
// The FP16 window [o + Q, T) holds at most residual + group - 1 tokens: residual / 32
// + 1 chunks of 32 tokens, plus one chunk for an attention sink; four chunks per
// decode workgroup.
constexpr int kWindowChunksPerBlock = 4;
constexpr int kMaxWindowBlocks = (kMaxResidual / kGroup + 2 + kWindowChunksPerBlock - 1) / kWindowChunksPerBlock;

// Per-sequence record kept on the device and rewritten by every append:
// tokens before the append, tokens appended, quantized tokens before and after.
struct SeqDesc {
  int32_t t_old;
  int32_t n_new;
  int32_t q_old;
  int32_t q_new;
};

// Per-sequence records of one append, passed to its kernels by value when the batch
// is small (no host-to-device copy), otherwise read from the device array `dev`.
// With `inl_valid`, the window-write kernel also stores them to `state`, the array
// the decode kernel reads.
constexpr int kInlineSeqs = 64;
struct SeqArgs {
  SeqDesc inl[kInlineSeqs];
  const SeqDesc* dev;
  SeqDesc* state;
  int inl_valid;
};

// The record of sequence b (wave-uniform). The inline copy is read on its own from
// the kernel arguments, so that it comes through scalar loads; choosing between the
// two sources by address made it a vector load from a generic address, which the
// workgroup waited on before its first loads.
__device__ inline SeqDesc seq_record(const SeqArgs& s, const SeqDesc* dev, int b) {
  SeqDesc r = s.inl[s.inl_valid ? b : 0];
  if (!s.inl_valid) {
    // a load of another kind, so that it is not merged with the one above
    typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
    const i32x4 d = __builtin_nontemporal_load(reinterpret_cast<const i32x4*>(dev) + b);
    r = SeqDesc{d[0], d[1], d[2], d[3]};
  }
  return r;
}

// An append folded into a decode launch (caches without rotation): the FP16-window
// workgroups read the appended tokens from k / v ([B][n_max][Hkv][128] fp16), write
// the tokens that stay in the window to the ring, and with inline records store them
// as the sequences' state. Every workgroup takes the sequence lengths from `seq`
// (inline) or the device state (uploaded records).
struct AppendArgs {
  int32_t pending;
  const void* k;
  const void* v;
  int32_t n_max;
  SeqArgs seq;
};

// Decode work split: every kv-head of sequence b gets n_b split workgroups of
// groups_per_split groups each. With use_prefix (batch at most kInlineSeqs) the
// sequences are taken in the order seq[0], seq[1], ... (longest first) and
// prefix[p] = n_seq[0] + ... + n_seq[p-1]; count[b] = n_b. Otherwise every sequence
// has n_b = uniform, in index order. Partials of (sequence, query head) sit at
// `pstride` slots: n_b splits, then the FP16 window's.
//
// With `older_weight` > 0 (one round of equal sequences, two workgroups per compute
// unit) the grid is split-major: the first half of the split workgroups, which the
// dispatcher places first on every compute unit and which then get its issue
// priority, are the lower half of every head's splits, and each of them takes
// older_weight times the groups of a split in the upper half.
struct SplitPlan {
  int32_t prefix[kInlineSeqs + 1];
  int32_t seq[kInlineSeqs];
  int32_t count[kInlineSeqs];
  int32_t use_prefix;
  int32_t uniform;
  int32_t pstride;
  float older_weight;
};

// Where the packed group blocks live. Contiguous caches: [B][Hkv][gcap][GB].
// Paged caches: a pool of pages, each [Hkv][P][GB] for P consecutive groups of one
// sequence; table[b][g / P] names the page of group g of sequence b.
struct GroupStore {
  uint8_t* blocks;
  const int32_t* table;  // [B][max_pages]; null for a contiguous cache
  long long gcap;
  int Hkv, P, pshift, max_pages, gb;  // P = 2^pshift groups per page
  __host__ __device__ size_t offset(int b, int h, long long g, int page) const {
    if (!table) return ((size_t(b) * Hkv + h) * size_t(gcap) + size_t(g)) * size_t(gb);
    return ((size_t(page) * Hkv + h) * size_t(P) + size_t(g & (P - 1))) * size_t(gb);
  }
  // Device side: looks the page up in the table. The table does not change while a
  // kernel runs, so it is read through the constant address space: a wave-uniform
  // index then gives one scalar load, whatever else the kernel does with memory
  // (read as a generic global load, the entry came through a vector load that waited
  // behind the group loads in flight).
  __device__ uint8_t* at(int b, int h, long long g) const {
    typedef __attribute__((address_space(4))) const int32_t* const_i32p;
    const int page =
        table ? __builtin_amdgcn_readfirstlane(((const_i32p)table)[size_t(b) * max_pages + size_t(g >> pshift)]) : 0;
    return blocks + offset(b, h, g, page);
  }
};

struct Layout {
  int32_t B, Hq, Hkv, bits, R, W;  // W = R + G window slots (token t >= o in slot t % W)
  int32_t sink;                     // 1: token 0 is an attention sink, kept in ring slot W
  int32_t RS;                       // ring slots per (b, h): W + sink
  int32_t rope;                     // 1: keys are pre-RoPE, rotated after dequantization
  int32_t rope_entries;             // rows of the rotary table (group start positions)
  int32_t P;                        // paged caches: groups per page (0: contiguous)
  int32_t max_pages;                // paged caches: table entries per sequence
  int64_t pool_pages;               // paged caches: pages in the pool
  int64_t gcap;                     // group blocks per (b, h)
  size_t group_bytes;
  int32_t max_splits;
  int32_t win_blocks;  // FP16-window decode workgroups per (b, h)
  size_t seq_off, table_off, blocks_off, ringk_off, ringv_off, part_off;
  size_t rope_off, ropein_off;  // rotary tables (pre-RoPE caches): [rope_entries][128], [32][128] fp32
  size_t total;
};

// Launchers (return hipGetLastError() of the launch).
// The group store of a cache laid out by L at base.
inline GroupStore group_store(const Layout& L, uint8_t* base) {
  GroupStore s;
  s.blocks = base + L.blocks_off;
  s.table = L.P ? reinterpret_cast<const int32_t*>(base + L.table_off) : nullptr;
  s.gcap = L.gcap;
  s.Hkv = L.Hkv;
  s.P = L.P > 0 ? L.P : 1;
  s.pshift = 0;
  while ((1 << s.pshift) < s.P) s.pshift++;
  s.max_pages = L.max_pages;
  s.gb = int(L.group_bytes);
  return s;
}

hipError_t launch_flush(const Layout& L, uint8_t* base, const SeqArgs& seq, const void* k,
                        const void* v, int32_t n_max, int32_t max_flush_groups, int rotate,
                        hipStream_t stream);
hipError_t launch_ring_write(const Layout& L, uint8_t* base, const SeqArgs& seq, const void* k,
                             const void* v, int32_t n_max, int32_t max_ring_tokens, int rotate,
                             hipStream_t stream);
// Workgroups of the decode split kernel that fit on one compute unit of the current
// device at once, and the device's compute units.
int decode_blocks_per_cu(int bits, int hg, int rope);
int device_compute_units();
hipError_t launch_rope_tables(const Layout& L, uint8_t* base, double rope_base, hipStream_t stream);
hipError_t launch_decode(const Layout& L, uint8_t* base, const SeqDesc* seq, const AppendArgs& app,
                         const void* q, float* out, int32_t groups_per_split, const SplitPlan& plan,
                         float scale_log2, int rotate, hipStream_t stream, hipEvent_t prof_start,
                         hipEvent_t prof_stop);

// Merge the partials of every (sequence, query head), laid out [B][Hq][pstride][130]:
// sequence b has nsplit_b + wblocks of them (nsplit_b from the plan).
hipError_t launch_combine(const float* part, float* out, int Hq, int B, const SplitPlan& plan, int wblocks,
                          hipStream_t stream);

// Comparison kernels: streaming read of a buffer; decode over a plain FP16 cache
// [B][Hkv][t_cap][128] (partials [B][Hq][nsplit][130] in `part`).
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* fold, int blocks, hipStream_t stream);
hipError_t launch_fp16_decode(const void* k, const void* v, const int32_t* lens, long long t_cap, int B, int Hq,
                              int Hkv, float scale_log2, const void* q, float* out, float* part, int nsplit,
                              int cps, hipStream_t stream);
constexpr int kFp16MaxSplits = 1024;
constexpr int kMaxStreamWorkgroups = 1 << 16;  // streaming-read probe: one fold word per workgroup
// The FP16-cache decode's static scratch (partials of the variant that allocates
// nothing): 4 MiB per GPU, room for 8065 partials of 520 bytes.
constexpr size_t kFp16ScratchBytes = size_t(4) << 20;
// Device address of that scratch on the current device (looked up once per device).
hipError_t fp16_scratch(void** ptr);

}  // namespace kvq
