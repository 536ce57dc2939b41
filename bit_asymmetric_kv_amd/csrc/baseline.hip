// Comparison kernels measured beside the quantized decode path:
//  * a streaming read of a device buffer, the achievable HBM read bandwidth that
//    the decode kernel's effective bandwidth is set against;
//  * decode attention over a plain FP16 KV cache, the full-precision decode the
//    pages compare low-bit caches with (FlashAttention-style decoding over the
//    whole cache: "Read What Matters", the RDKV abstract; decode is bound by
//    reading the cache, "KV cache quantization: putting the bits in the cached
//    vectors", the KIVI abstract).
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include <mutex>

#include "kvq_internal.h"

// Split partials of the FP16-cache decode for callers that cannot allocate: one
// copy per GPU, held until the process ends. In host code this name is only a
// stand-in for the symbol; its device address comes from hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[kvq::kFp16ScratchBytes];

namespace kvq {
namespace {

constexpr int kD = kHeadDim;
constexpr int kChunk = 32;
constexpr int kWaves = 4;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef _Float16 half4v __attribute__((ext_vector_type(4)));

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Streaming loads of cache rows that a decode call reads once: non-temporal, so the
// rows do not displace what is reused (8 % faster FP16-cache decode at 128K tokens).
__device__ inline uint4 stream_load16(const __half* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}
__device__ inline uint2 stream_load8(const __half* p) {
  return __builtin_bit_cast(uint2, __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p)));
}

// Reads every 16-byte word of buf[0, n16) once (grid-stride, four words in flight
// per thread, nontemporal loads: the data is not reused), folds the words with xor
// and stores workgroup i's fold in fold[i], so the loads stay live without any
// atomic (one word per workgroup: no serialized read-modify-write at the end).
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ buf, size_t n16,
                                                          uint32_t* __restrict__ fold) {
  uint32_t acc = 0;
  const size_t stride = size_t(gridDim.x) * blockDim.x;
  size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(buf + i), b = __builtin_nontemporal_load(buf + i + stride),
                c = __builtin_nontemporal_load(buf + i + 2 * stride),
                d = __builtin_nontemporal_load(buf + i + 3 * stride);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^
           d[3];
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(buf + i);
    acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
  }
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  __shared__ uint32_t red[4];
  if (threadIdx.x % 64 == 0) red[threadIdx.x / 64] = acc;
  __syncthreads();
  if (threadIdx.x == 0) fold[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

struct Fp16Args {
  const __half* k;
  const __half* v;
  const int32_t* lens;
  const __half* q;
  float* part;
  long long t_cap;
  int Hq, Hkv, nsplit, cps;  // cps: 32-token chunks per workgroup
  float scale_log2;
};

// One workgroup per (split of cps chunks of 32 tokens, kv-head, sequence); its four
// waves take the split's chunks in turn (wave w: chunks w, w + 4, ...). A wave holds
// one chunk in registers and issues the next chunk's key loads as soon as its score
// MFMAs have read the keys and its value loads as soon as the weighted sum has read
// the values; the many resident waves keep enough loads in flight.
//
// Scores: an MFMA 16x16x32 f16 contraction over channels with the keys as A (token
// rows straight from the cache, exact fp16) and the query as B (exact fp16), one
// MFMA column per head (copies fill the 16 columns), fp32 accumulation; the softmax
// scale is applied to the fp32 scores. Lane (column c, row block kb) then holds the
// scores of head c % HG for tokens 4 kb + i and 16 + 4 kb + i (i < 4).
// Weighted values: lane l accumulates channels 4 (l % 32) .. + 3 over the chunk's
// tokens 2 i + l / 32 (8 bytes per token: a half-wave reads one 256-byte row) for
// every head, with fused multiply-adds in fp32; the softmax weights of all heads
// reach the lanes through the wave's shared memory. The two half-waves' sums are
// added once, after the wave's last chunk.
template <int HG>
__global__ __launch_bounds__(256, HG == 8 ? 1 : 2) void fp16_split_kernel(Fp16Args a) {
  __shared__ float pst[kWaves][kChunk][HG];               // softmax weights of the current chunk
  __shared__ float wpart[kWaves][HG][kPartialStride];     // per-wave partials
  const int split = blockIdx.x % a.nsplit;
  const int h = (blockIdx.x / a.nsplit) % a.Hkv;
  const int b = blockIdx.x / (a.nsplit * a.Hkv);
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int col = lane % 16, kb = lane / 16, hc = col % HG;
  const int vc = lane % 32, vh = lane / 32;  // value channels 4 vc .. + 3, tokens 2 i + vh
  const int T = int(min<long long>(a.lens[b], a.t_cap));
  const int nch = (T + kChunk - 1) / kChunk;
  const int c0 = split * a.cps, c1 = min(nch, c0 + a.cps);
  const int len = max(0, c1 - c0);
  const int n = __builtin_amdgcn_readfirstlane(max(0, (len - wave + kWaves - 1) / kWaves));
  const size_t row0 = (size_t(b) * a.Hkv + h) * size_t(a.t_cap);
  const __half* kbase = a.k + row0 * kD;
  const __half* vbase = a.v + row0 * kD;

  auto chunk_start = [&](int r) { return (c0 + wave + kWaves * r) * kChunk; };
  uint4 kr[8];   // kr[2 kc + tile]: key row 16 tile + col, channels 32 kc + 8 kb .. + 7
  uint2 vr[16];  // vr[i]: value row 2 i + vh, channels 4 vc .. + 3
  auto load_keys = [&](int r) {
    const int t0 = chunk_start(r);
    for (int tile = 0; tile < 2; tile++)
      for (int kc = 0; kc < 4; kc++) {
        const int t = min(t0 + 16 * tile + col, T - 1);  // rows past the end re-read the last one
        kr[2 * kc + tile] = stream_load16(kbase + size_t(t) * kD + 32 * kc + 8 * kb);
      }
  };
  auto load_values = [&](int r) {
    const int t0 = chunk_start(r);
    for (int i = 0; i < 16; i++) {
      const int t = min(t0 + 2 * i + vh, T - 1);
      vr[i] = stream_load8(vbase + size_t(t) * kD + 4 * vc);
    }
  };
  if (n > 0) {
    load_keys(0);
    load_values(0);
  }

  // query of head hc as the MFMA B operand (channels 32 kc + 8 kb .. + 7)
  half8 qb[4];
  {
    const __half* qrow = a.q + (size_t(b) * a.Hq + h * HG + hc) * kD;
    for (int kc = 0; kc < 4; kc++)
      qb[kc] = __builtin_bit_cast(half8, *reinterpret_cast<const uint4*>(qrow + 32 * kc + 8 * kb));
  }

  float m[HG];         // running max per head (log2 units), the same in every lane
  float l_col = 0.0f;  // sum of this lane's weights of head hc
  float o[HG][4];      // this lane's channels, over its half-wave's tokens
  for (int hh = 0; hh < HG; hh++) {
    m[hh] = -INFINITY;
    for (int c = 0; c < 4; c++) o[hh][c] = 0.0f;
  }

  for (int r = 0; r < n; r++) {
    const int t0 = chunk_start(r);
    float4v s0 = {0.0f, 0.0f, 0.0f, 0.0f}, s1 = s0;
    for (int kc = 0; kc < 4; kc++) {
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, kr[2 * kc]), qb[kc], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, kr[2 * kc + 1]), qb[kc], s1, 0, 0, 0);
    }
    if (r + 1 < n) load_keys(r + 1);
    float x[8];
    float mx = -INFINITY;
    for (int i = 0; i < 8; i++) {
      const int tk = i < 4 ? 4 * kb + i : 16 + 4 * kb + (i - 4);
      const float sv = i < 4 ? s0[i] : s1[i - 4];
      x[i] = t0 + tk < T ? sv * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, x[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));  // chunk max of head hc (every chunk holds a valid token)
    float alpha[HG];
    bool grew = false;
    for (int hh = 0; hh < HG; hh++) {
      const float mh = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mx), hh));
      const float mn = fmaxf(m[hh], mh);
      alpha[hh] = m[hh] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m[hh] - mn);
      grew = grew || mn != m[hh];
      m[hh] = mn;
    }
    float mcol = m[0], acol = alpha[0];
    for (int hh = 1; hh < HG; hh++) {
      mcol = hc == hh ? m[hh] : mcol;
      acol = hc == hh ? alpha[hh] : acol;
    }
    float ps = 0.0f;
    for (int i = 0; i < 8; i++) {
      const int tk = i < 4 ? 4 * kb + i : 16 + 4 * kb + (i - 4);
      x[i] = __builtin_amdgcn_exp2f(x[i] - mcol);  // non-positive argument; -inf gives 0
      ps += x[i];
      if (col < HG) pst[wave][tk][col] = x[i];
    }
    l_col = l_col * acol + ps;
    if (grew)
      for (int hh = 0; hh < HG; hh++)
        for (int c = 0; c < 4; c++) o[hh][c] *= alpha[hh];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int i = 0; i < 16; i++) {
      // at most four tokens' weights in registers at a time (the compiler would
      // otherwise read all 16 x HG of them up front)
      if (i % 4 == 0) asm volatile("" ::: "memory");
      float pw[HG];
      for (int hh = 0; hh < HG; hh++) pw[hh] = pst[wave][2 * i + vh][hh];
      const half4v v4 = __builtin_bit_cast(half4v, vr[i]);
      for (int c = 0; c < 4; c++) {
        const float vf = float(v4[c]);
        for (int hh = 0; hh < HG; hh++) o[hh][c] = __builtin_fmaf(vf, pw[hh], o[hh][c]);
      }
    }
    // the next chunk's values go into the registers this chunk's have just left
    asm volatile("" ::: "memory");
    if (r + 1 < n) load_values(r + 1);
    // the weights are read before the next chunk overwrites them
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // sums over the two half-waves (values) and the four row blocks (weights); lanes
  // 0..31 write the wave's partial
  for (int hh = 0; hh < HG; hh++)
    for (int c = 0; c < 4; c++) o[hh][c] += __shfl_xor(o[hh][c], 32);
  float lt = l_col + __shfl_xor(l_col, 16);
  lt += __shfl_xor(lt, 32);
  if (vh == 0) {
    for (int hh = 0; hh < HG; hh++)
      for (int c = 0; c < 4; c++) wpart[wave][hh][2 + 4 * vc + c] = o[hh][c];
  }
  if (kb == 0 && col < HG) {
    float mc = m[0];
    for (int hh = 1; hh < HG; hh++) mc = col == hh ? m[hh] : mc;
    wpart[wave][col][0] = mc;
    wpart[wave][col][1] = lt;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < HG * kPartialStride; idx += blockDim.x) {
    const int hh = idx / kPartialStride, c = idx % kPartialStride;
    float M = -INFINITY;
    for (int w = 0; w < kWaves; w++) M = fmaxf(M, wpart[w][hh][0]);
    float res = 0.0f;
    if (c == 0) {
      res = M;
    } else if (M != -INFINITY) {
      for (int w = 0; w < kWaves; w++)
        if (wpart[w][hh][0] != -INFINITY) res += wpart[w][hh][c] * __builtin_amdgcn_exp2f(wpart[w][hh][0] - M);
    }
    a.part[((size_t(b) * a.Hq + h * HG + hh) * a.nsplit + split) * kPartialStride + c] = res;
  }
}

template <int HG>
hipError_t launch_fp16(const Fp16Args& a, int B, hipStream_t stream) {
  hipLaunchKernelGGL((fp16_split_kernel<HG>), dim3(a.nsplit * a.Hkv * B), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t fp16_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    // first use on this device (the current one): its own copy of the array
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* fold, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, stream, static_cast<const u32x4*>(buf),
                     bytes / 16, fold);
  return hipGetLastError();
}

hipError_t launch_fp16_decode(const void* k, const void* v, const int32_t* lens, long long t_cap, int B, int Hq,
                              int Hkv, float scale_log2, const void* q, float* out, float* part, int nsplit,
                              int cps, hipStream_t stream) {
  Fp16Args a;
  a.k = static_cast<const __half*>(k);
  a.v = static_cast<const __half*>(v);
  a.lens = lens;
  a.q = static_cast<const __half*>(q);
  a.part = part;
  a.t_cap = t_cap;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.nsplit = nsplit;
  a.cps = cps;
  a.scale_log2 = scale_log2;
  const int hg = Hq / Hkv;
  hipError_t e = hg == 1 ? launch_fp16<1>(a, B, stream)
                 : hg == 2 ? launch_fp16<2>(a, B, stream)
                 : hg == 4 ? launch_fp16<4>(a, B, stream)
                           : launch_fp16<8>(a, B, stream);
  if (e != hipSuccess) return e;
  SplitPlan plan{};
  plan.use_prefix = 0;
  plan.uniform = nsplit;
  plan.pstride = nsplit;
  return launch_combine(part, out, Hq, B, plan, 0, stream);
}

}  // namespace kvq
