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

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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

// Online-softmax state of one wave for HG query heads: max m and sum l (log2
// domain, identical in every lane) and the unnormalized output of channels
// 2 lane, 2 lane + 1.
template <int HG>
struct Fp16State {
  float m[HG], l[HG], o0[HG], o1[HG];
};

// Attention over tokens [t0, t0 + cnt) (cnt in 1..32) of one (sequence, kv-head):
// lane l scores token l % 32 over channel half l / 32, then every lane accumulates
// its two channels over the chunk's tokens.
template <int HG>
__device__ void fp16_chunk(const __half* krow0, const __half* vrow0, int cnt, const float (*qf)[kD],
                           Fp16State<HG>& st, int lane) {
  const int tl = lane % 32, hf = lane / 32;
  const bool kval = tl < cnt;
  uint4 kr[8];
  {
    const uint4* kp = reinterpret_cast<const uint4*>(krow0 + size_t(kval ? tl : 0) * kD + 64 * hf);
    for (int i = 0; i < 8; i++) kr[i] = kp[i];
  }
  uint32_t vr[kChunk];
  for (int t = 0; t < kChunk; t++)
    vr[t] = *reinterpret_cast<const uint32_t*>(vrow0 + size_t(t < cnt ? t : 0) * kD + 2 * lane);
  float x[HG];
  for (int hh = 0; hh < HG; hh++) x[hh] = 0.0f;
  for (int i = 0; i < 8; i++) {
    // The query rows stay in shared memory: without this barrier the compiler hoists
    // all of their loads out of the chunk loop into registers.
    asm volatile("" ::: "memory");
    const half8 k8 = __builtin_bit_cast(half8, kr[i]);
    for (int e = 0; e < 8; e++) {
      const float kv = float(k8[e]);
      for (int hh = 0; hh < HG; hh++) x[hh] = __builtin_fmaf(qf[hh][64 * hf + 8 * i + e], kv, x[hh]);
    }
  }
  float p[HG];
  for (int hh = 0; hh < HG; hh++) {
    const float xs = x[hh] + __shfl_xor(x[hh], 32);
    const float sc = kval ? xs : -INFINITY;
    float cm = sc;
    for (int off = 16; off > 0; off >>= 1) cm = fmaxf(cm, __shfl_xor(cm, off));
    const float mn = fmaxf(st.m[hh], cm);
    const float alpha = st.m[hh] == -INFINITY ? 0.0f : exp2f(st.m[hh] - mn);
    p[hh] = kval ? exp2f(sc - mn) : 0.0f;
    float ls = p[hh];
    for (int off = 16; off > 0; off >>= 1) ls += __shfl_xor(ls, off);
    st.l[hh] = st.l[hh] * alpha + ls;
    st.o0[hh] *= alpha;
    st.o1[hh] *= alpha;
    st.m[hh] = mn;
  }
  for (int t = 0; t < kChunk; t++) {
    if (t < cnt) {
      const half2v vv = __builtin_bit_cast(half2v, vr[t]);
      const float v0 = float(vv[0]), v1 = float(vv[1]);
      for (int hh = 0; hh < HG; hh++) {
        const float pt = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, p[hh]), t));
        st.o0[hh] = __builtin_fmaf(pt, v0, st.o0[hh]);
        st.o1[hh] = __builtin_fmaf(pt, v1, st.o1[hh]);
      }
    }
  }
}

// One workgroup per (split of cps chunks, kv-head, sequence); its four waves take
// contiguous quarters of the split, and their states are merged into the split's
// partial (m, l, o[128]) per query head.
template <int HG>
__global__ __launch_bounds__(256) void fp16_split_kernel(Fp16Args a) {
  __shared__ float qf[HG][kD];
  __shared__ float wpart[kWaves][HG][kPartialStride];
  const int split = blockIdx.x % a.nsplit;
  const int h = (blockIdx.x / a.nsplit) % a.Hkv;
  const int b = blockIdx.x / (a.nsplit * a.Hkv);
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int T = int(min<long long>(a.lens[b], a.t_cap));
  const int nch = (T + kChunk - 1) / kChunk;

  for (int e = threadIdx.x; e < HG * kD; e += blockDim.x)
    qf[e / kD][e % kD] = __half2float(a.q[(size_t(b) * a.Hq + h * HG + e / kD) * kD + e % kD]) * a.scale_log2;
  __syncthreads();

  const int c0 = split * a.cps, c1 = min(nch, c0 + a.cps);
  const int per = (max(0, c1 - c0) + kWaves - 1) / kWaves;
  const int wc0 = c0 + wave * per, wc1 = min(c1, wc0 + per);
  Fp16State<HG> st;
  for (int hh = 0; hh < HG; hh++) {
    st.m[hh] = -INFINITY;
    st.l[hh] = st.o0[hh] = st.o1[hh] = 0.0f;
  }
  const size_t row0 = (size_t(b) * a.Hkv + h) * size_t(a.t_cap);
  for (int c = wc0; c < wc1; c++) {
    const int t0 = c * kChunk;
    fp16_chunk<HG>(a.k + (row0 + t0) * kD, a.v + (row0 + t0) * kD, min(kChunk, T - t0), qf, st, lane);
  }
  for (int hh = 0; hh < HG; hh++) {
    wpart[wave][hh][2 + 2 * lane] = st.o0[hh];
    wpart[wave][hh][3 + 2 * lane] = st.o1[hh];
    if (lane == 0) {
      wpart[wave][hh][0] = st.m[hh];
      wpart[wave][hh][1] = st.l[hh];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < HG * kPartialStride; idx += blockDim.x) {
    const int hh = idx / kPartialStride, c = idx % kPartialStride;
    float M = -INFINITY;
    for (int w = 0; w < kWaves; w++) M = fmaxf(M, wpart[w][hh][0]);
    float r = 0.0f;
    if (c == 0) {
      r = M;
    } else if (M != -INFINITY) {
      for (int w = 0; w < kWaves; w++)
        if (wpart[w][hh][0] != -INFINITY) r += wpart[w][hh][c] * exp2f(wpart[w][hh][0] - M);
    }
    a.part[((size_t(b) * a.Hq + h * HG + hh) * a.nsplit + split) * kPartialStride + c] = r;
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
