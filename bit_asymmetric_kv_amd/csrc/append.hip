// Append path: FP16 residual window writes and group quantize + pack.
//
// The residual rule keeps the most recent R tokens in FP16 ("The Asymmetric
// Key-Value Cache Compression Framework", In practice) and moves older tokens to
// the quantized store one 32-token group at a time, appended along the token
// dimension ("KV cache quantization: putting the bits in the cached vectors",
// full-text-skim notes on KIVI's grouped/residual streaming). Keys are quantized
// per channel over the group's tokens, values per token over 32-channel groups
// (same pages, Summary / Method).
//
// Every floating-point step of the quantizer is a single fp32 rounding with no
// contraction, so the stored codes, scales and zero-points are reproducible bit for
// bit from the formula documented in kvq.h.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "kvq_internal.h"

#pragma clang fp contract(off)

namespace kvq {
namespace {

constexpr int kD = kHeadDim;
constexpr int kG = kGroup;

// fp32 value of 1/sqrt(128) = sqrt(2)/16, correctly rounded.
constexpr float kInvSqrt128 = 0x1.6a09e6p-4f;

// Normalized Walsh-Hadamard transform of `nrows` rows of 128 fp32 values held in
// shared memory (row stride `stride`), natural (Sylvester) order: stages with
// half-width 1, 2, ..., 64, each butterfly (a, b) -> (a + b, a - b) in fp32, then a
// multiply by fp32(1/sqrt(128)) and a round trip through fp16, which is how a
// rotated key is stored. Rows with rot[row] == 0 are left untouched. Must be
// called by every thread of the block.
__device__ void rotate_rows_to_fp16(float* x, int stride, int nrows, const int* rot) {
  const int pairs = nrows * (kD / 2);
  for (int h = 1; h < kD; h <<= 1) {
    for (int p = threadIdx.x; p < pairs; p += blockDim.x) {
      int row = p / (kD / 2);
      if (!rot[row]) continue;
      int j = p % (kD / 2);
      int ia = (j / h) * (2 * h) + (j % h);
      float* r = x + row * stride;
      float a = r[ia], b = r[ia + h];
      r[ia] = a + b;
      r[ia + h] = a - b;
    }
    __syncthreads();
  }
  for (int e = threadIdx.x; e < nrows * kD; e += blockDim.x) {
    int row = e / kD;
    if (!rot[row]) continue;
    float* r = x + row * stride + (e % kD);
    float y = *r * kInvSqrt128;
    // Keep the fp32 rounding of the product: without this the compiler fuses the
    // multiply and the fp16 conversion into one mixed-precision op that rounds once.
    asm volatile("" : "+v"(y));
    *r = __half2float(__float2half_rn(y));
  }
  __syncthreads();
}

struct QuantOut {
  __half s, z;
};

// Asymmetric uniform quantization of the values x[0..31] (stride `step`):
// fp32 range / (2^bits - 1), fp16 scale and zero-point, codes from the stored
// fp16 scale with round-half-even and a clamp to [0, 2^bits - 1].
template <int BITS>
__device__ QuantOut quantize32(const float* x, int step, uint8_t* codes, int cstep) {
  const float levels = float((1 << BITS) - 1);
  float mn = x[0], mx = x[0];
  for (int i = 1; i < kG; i++) {
    float v = x[i * step];
    mn = fminf(mn, v);
    mx = fmaxf(mx, v);
  }
  float s32 = (mx - mn) / levels;
  __half s16 = __float2half_rn(s32);
  __half z16 = __float2half_rn(mn);
  float sf = __half2float(s16);
  float zf = __half2float(z16);
  if (sf == 0.0f) {
    for (int i = 0; i < kG; i++) codes[i * cstep] = 0;
  } else {
    float inv = 1.0f / sf;
    for (int i = 0; i < kG; i++) {
      float d = x[i * step] - zf;
      float r = __builtin_rintf(d * inv);
      r = fminf(fmaxf(r, 0.0f), levels);
      codes[i * cstep] = uint8_t(r);
    }
  }
  return {s16, z16};
}

// Token index of value-code slot s held by lane row kb.
__device__ inline int value_token(int kb, int s) { return s < 4 ? 4 * kb + s : 16 + 4 * kb + (s - 4); }

template <int BITS>
__global__ __launch_bounds__(256) void flush_kernel(uint8_t* __restrict__ blocks, const __half* __restrict__ ringk,
                                                    const __half* __restrict__ ringv, const SeqArgs seq,
                                                    const __half* __restrict__ kin, const __half* __restrict__ vin,
                                                    int Hkv, int W, int RS, int sink, long long gcap, int n_max,
                                                    int rotate) {
  constexpr int CB = kG * kD * BITS / 8;  // bytes of one code section
  constexpr int GB = 2 * CB + 1024;
  __shared__ float xk[kG][kD + 1];
  __shared__ float xv[kG][kD + 1];
  __shared__ uint8_t ck[kG][kD];
  __shared__ uint8_t cv[kG][kD];
  __shared__ int from_input[kG];

  const int h = blockIdx.y, b = blockIdx.z;
  const SeqDesc sd = seq.inl_valid ? seq.inl[b] : seq.dev[b];
  const int nflush = (sd.q_new - sd.q_old) / kG;
  if (int(blockIdx.x) >= nflush) return;
  const int g = sd.q_old / kG + blockIdx.x;
  const int t0 = sink + g * kG;  // with an attention sink, group g starts at token 1 + 32 g
  const size_t bh = size_t(b) * Hkv + h;

  if (threadIdx.x < kG) from_input[threadIdx.x] = (t0 + int(threadIdx.x) >= sd.t_old) ? 1 : 0;
  for (int e = threadIdx.x; e < kG * kD; e += blockDim.x) {
    int i = e / kD, d = e % kD;
    int t = t0 + i;
    __half kv, vv;
    if (t < sd.t_old) {
      size_t off = (bh * RS + size_t(t % W)) * kD + d;
      kv = ringk[off];
      vv = ringv[off];
    } else {
      size_t off = ((size_t(b) * n_max + (t - sd.t_old)) * Hkv + h) * kD + d;
      kv = kin[off];
      vv = vin[off];
    }
    xk[i][d] = __half2float(kv);
    xv[i][d] = __half2float(vv);
  }
  __syncthreads();
  if (rotate) rotate_rows_to_fp16(&xk[0][0], kD + 1, kG, from_input);

  __shared__ __half ks[kD], kz[kD], vs[kD], vz[kD];
  if (threadIdx.x < kD) {
    int d = threadIdx.x;  // keys: one channel over the group's 32 tokens
    QuantOut r = quantize32<BITS>(&xk[0][d], kD + 1, &ck[0][d], kD);
    ks[d] = r.s;
    kz[d] = r.z;
  } else {
    int idx = threadIdx.x - kD;  // values: one token, one 32-channel group
    int i = idx / 4, j = idx % 4;
    QuantOut r = quantize32<BITS>(&xv[i][j * kG], 1, &cv[i][j * kG], 1);
    int kb = (i % 16) / 4, s = 4 * (i / 16) + i % 4;
    int vi = (kb * 4 + j) * 8 + s;
    vs[vi] = r.s;
    vz[vi] = r.z;
  }
  __syncthreads();

  uint8_t* blk = blocks + (bh * size_t(gcap) + g) * GB;
  uint32_t* kw = reinterpret_cast<uint32_t*>(blk);
  uint32_t* vw = reinterpret_cast<uint32_t*>(blk + CB);
  constexpr int NW = CB / 4;
  for (int w = threadIdx.x; w < NW; w += blockDim.x) {
    uint32_t kword = 0, vword = 0;
    if (BITS == 2) {
      int l = w / 4, ohi = w % 4;
      for (int par = 0; par < 2; par++) {
        int o = 2 * ohi + par;
        for (int s = 0; s < 8; s++) {
          int bit = 8 * (s / 2) + 4 * (s % 2) + 2 * par;
          int ki = 16 * (o % 2) + l % 16, kd = 32 * (o / 2) + 8 * (l / 16) + s;
          int vd = 16 * o + l % 16, vi = value_token(l / 16, s);
          kword |= uint32_t(ck[ki][kd]) << bit;
          vword |= uint32_t(cv[vi][vd]) << bit;
        }
      }
    } else {
      int o = 4 * (w / 256) + w % 4, l = (w % 256) / 4;
      for (int s = 0; s < 8; s++) {
        int bit = 8 * (s % 4) + 4 * (s / 4);
        int ki = 16 * (o % 2) + l % 16, kd = 32 * (o / 2) + 8 * (l / 16) + s;
        int vd = 16 * o + l % 16, vi = value_token(l / 16, s);
        kword |= uint32_t(ck[ki][kd]) << bit;
        vword |= uint32_t(cv[vi][vd]) << bit;
      }
    }
    kw[w] = kword;
    vw[w] = vword;
  }
  __half* sz = reinterpret_cast<__half*>(blk + 2 * CB);
  if (threadIdx.x < kD) {
    int d = threadIdx.x;
    sz[d] = ks[d];
    sz[kD + d] = kz[d];
    sz[2 * kD + d] = vs[d];
    sz[3 * kD + d] = vz[d];
  }
}

// One block per (appended token that stays in FP16, kv-head, sequence). Window
// token t (t >= o) goes to ring slot t % W; an attention sink (token 0, appended by
// the first append of the sequence) goes to slot W and takes block 0.
__global__ __launch_bounds__(128) void ring_write_kernel(__half* __restrict__ ringk, __half* __restrict__ ringv,
                                                         const SeqArgs seq, const __half* __restrict__ kin,
                                                         const __half* __restrict__ vin, int Hkv, int W, int RS,
                                                         int sink, int n_max, int rotate) {
  __shared__ float row[kD];
  __shared__ int one;
  const int h = blockIdx.y, b = blockIdx.z;
  const SeqDesc sd = seq.inl_valid ? seq.inl[b] : seq.dev[b];
  if (seq.inl_valid && blockIdx.x == 0 && h == 0 && threadIdx.x == 0) seq.state[b] = sd;
  const int t_new = sd.t_old + sd.n_new;
  const int sink_new = (sink && sd.t_old == 0 && sd.n_new > 0) ? 1 : 0;
  const int first = max(sd.t_old, sink + sd.q_new);
  const bool is_sink = sink_new && blockIdx.x == 0;
  const int t = is_sink ? 0 : first + int(blockIdx.x) - sink_new;
  if (t >= t_new) return;
  const int d = threadIdx.x;
  size_t in_off = ((size_t(b) * n_max + (t - sd.t_old)) * Hkv + h) * kD + d;
  size_t out_off = ((size_t(b) * Hkv + h) * RS + size_t(is_sink ? W : t % W)) * kD + d;
  ringv[out_off] = vin[in_off];
  if (!rotate) {
    ringk[out_off] = kin[in_off];
    return;
  }
  row[d] = __half2float(kin[in_off]);
  if (d == 0) one = 1;
  __syncthreads();
  rotate_rows_to_fp16(row, kD, 1, &one);
  ringk[out_off] = __float2half_rn(row[d]);
}

}  // namespace

hipError_t launch_flush(const Layout& L, uint8_t* base, const SeqArgs& seq, const void* k, const void* v,
                        int32_t n_max, int32_t max_flush_groups, int rotate, hipStream_t stream) {
  dim3 grid(max_flush_groups, L.Hkv, L.B);
  auto* blocks = base + L.blocks_off;
  auto* rk = reinterpret_cast<const __half*>(base + L.ringk_off);
  auto* rv = reinterpret_cast<const __half*>(base + L.ringv_off);
  auto* kin = static_cast<const __half*>(k);
  auto* vin = static_cast<const __half*>(v);
  if (L.bits == 2)
    hipLaunchKernelGGL(flush_kernel<2>, grid, dim3(256), 0, stream, blocks, rk, rv, seq, kin, vin, L.Hkv, L.W,
                       L.RS, L.sink, (long long)L.gcap, n_max, rotate);
  else
    hipLaunchKernelGGL(flush_kernel<4>, grid, dim3(256), 0, stream, blocks, rk, rv, seq, kin, vin, L.Hkv, L.W,
                       L.RS, L.sink, (long long)L.gcap, n_max, rotate);
  return hipGetLastError();
}

hipError_t launch_ring_write(const Layout& L, uint8_t* base, const SeqArgs& seq, const void* k, const void* v,
                             int32_t n_max, int32_t max_ring_tokens, int rotate, hipStream_t stream) {
  dim3 grid(max_ring_tokens, L.Hkv, L.B);
  hipLaunchKernelGGL(ring_write_kernel, grid, dim3(kD), 0, stream, reinterpret_cast<__half*>(base + L.ringk_off),
                     reinterpret_cast<__half*>(base + L.ringv_off), seq, static_cast<const __half*>(k),
                     static_cast<const __half*>(v), L.Hkv, L.W, L.RS, L.sink, n_max, rotate);
  return hipGetLastError();
}

}  // namespace kvq
