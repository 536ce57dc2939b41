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

// Token index of value-code slot s held by lane row kb.
__device__ inline int value_token(int kb, int s) { return s < 4 ? 4 * kb + s : 16 + 4 * kb + (s - 4); }

// Group flush with one wave per group, the data held in registers: the wave reads
// the group's 32 key rows and 32 value rows (FP16 window or appended input, 16 KB),
// quantizes keys per channel (lane l: channels 2l and 2l+1 over the 32 tokens) and
// values per token and 32-channel group (lane l: token l/4 and 16 + l/4, channel
// group l%4), puts the codes in shared memory and writes the packed block in the
// MFMA operand order. With rotation, keys read from the input go through the
// Walsh-Hadamard butterflies across lanes first (fp32 sums and differences, stage by
// stage as in rotate_rows_to_fp16).
//
// Asymmetric uniform quantization of 32 values: fp32 range / (2^bits - 1), fp16
// scale and zero-point, codes from the stored fp16 scale with round-half-even and a
// clamp to [0, 2^bits - 1].
template <int BITS>
__device__ inline QuantOut quantize_regs(const float* x, uint8_t* codes) {
  const float levels = float((1 << BITS) - 1);
  float mn = x[0], mx = x[0];
  for (int i = 1; i < kG; i++) {
    mn = fminf(mn, x[i]);
    mx = fmaxf(mx, x[i]);
  }
  const float s32 = (mx - mn) / levels;
  const __half s16 = __float2half_rn(s32);
  const __half z16 = __float2half_rn(mn);
  const float sf = __half2float(s16);
  const float zf = __half2float(z16);
  if (sf == 0.0f) {
    for (int i = 0; i < kG; i++) codes[i] = 0;
  } else {
    const float inv = 1.0f / sf;
    for (int i = 0; i < kG; i++) {
      const float d = x[i] - zf;
      float r = __builtin_rintf(d * inv);
      r = fminf(fmaxf(r, 0.0f), levels);
      codes[i] = uint8_t(r);
    }
  }
  return {s16, z16};
}

// ROT: keys are Walsh-Hadamard rotated (a template parameter, so that the rotation's
// registers do not lower the occupancy of the plain kernel).
template <int BITS, bool ROT>
__global__ __launch_bounds__(64) void flush_wave_kernel(const GroupStore store, const __half* __restrict__ ringk,
                                                        const __half* __restrict__ ringv, const SeqArgs seq,
                                                        const __half* __restrict__ kin,
                                                        const __half* __restrict__ vin, int Hkv, int W, int RS,
                                                        int sink, int n_max) {
  constexpr int CB = kG * kD * BITS / 8;  // bytes of one code section
  // key and value codes [token][channel]; with rotation the same bytes first hold the
  // rotated keys [token][channel] on their way to the per-channel layout
  // Key-code rows are padded by 4 bytes: the gather below reads one byte from each of
  // 16 token rows at once, which with 128-byte rows all fall in one bank.
  __shared__ union {
    struct {
      uint8_t ck[kG][kD + 4];
      uint8_t cv[kG][kD];
    } c;
    __half kt[kG][kD];
  } sm;
  auto& ck = sm.c.ck;
  auto& cv = sm.c.cv;
  auto& kt = sm.kt;
  __shared__ __half vsz[2][kD];   // value scales / zero-points in block order

  const int lane = threadIdx.x, h = blockIdx.y, b = blockIdx.z;
  // The record is the same for the whole wave: its fields go to scalar registers, so
  // that the row addresses below are wave-uniform arithmetic.
  const SeqDesc sdl = seq_record(seq, seq.dev, b);
  const int t_old = __builtin_amdgcn_readfirstlane(sdl.t_old);
  const int q_old = __builtin_amdgcn_readfirstlane(sdl.q_old);
  const int q_new = __builtin_amdgcn_readfirstlane(sdl.q_new);
  const int nflush = (q_new - q_old) / kG;
  if (int(blockIdx.x) >= nflush) return;
  const int g = q_old / kG + blockIdx.x;
  const int t0 = sink + g * kG;  // with an attention sink, group g starts at token 1 + 32 g
  const size_t bh = size_t(b) * Hkv + h;
  // Row of token t0 + i (0 <= i < 32): FP16 window slot (t0 + i) % W if it was appended
  // before, else input row. W = R + 32 >= 32, so the slots of the group's 32
  // consecutive tokens wrap around the window at most once. The input offset of row 0
  // is negative when the group starts inside the window; it is used only for rows
  // t >= t_old, whose offsets are not.
  const int s0 = t0 % W;
  const int64_t ring_off0 = (int64_t(bh) * RS + s0) * kD;
  const int64_t in_off0 = ((int64_t(b) * n_max + (t0 - t_old)) * Hkv + h) * kD;
  const int64_t in_step = int64_t(Hkv) * kD;
  auto row = [&](const __half* ring, const __half* in, int i) -> const __half* {
    if (t0 + i >= t_old) return in + (in_off0 + int64_t(i) * in_step);
    return ring + (ring_off0 + int64_t(s0 + i >= W ? i - W : i) * kD);
  };
  uint8_t* blk = store.at(b, h, g);

  // Every load of the group is issued before any arithmetic: 32 key words (channels
  // 2l, 2l+1 of each token; with rotation, lane l takes half l % 2 of token l / 2
  // instead) and the lane's two 64-byte value segments.
  uint32_t ku[kG];
  uint4 kr[8];
  if constexpr (ROT) {
    const uint4* src = reinterpret_cast<const uint4*>(row(ringk, kin, lane / 2) + 64 * (lane % 2));
    for (int q = 0; q < 8; q++) kr[q] = src[q];
  } else {
    for (int i = 0; i < kG; i++) ku[i] = *reinterpret_cast<const uint32_t*>(row(ringk, kin, i) + 2 * lane);
  }
  uint4 vu[2][4];
  for (int k = 0; k < 2; k++) {
    const uint4* src = reinterpret_cast<const uint4*>(row(ringv, vin, 16 * k + lane / 4) + kG * (lane % 4));
    for (int q = 0; q < 4; q++) vu[k][q] = src[q];
  }

  // Keys.
  {
    float x0[kG], x1[kG];
    if constexpr (ROT) {
      // Lane l rotates half l % 2 (channels 64 (l % 2) ...) of token t0 + l / 2: the
      // butterflies of half-width 1 ... 32 stay in its registers, half-width 64 pairs
      // it with lane l ^ 1; the rounded keys go through shared memory back to the
      // per-channel layout. Window rows are stored rotated already.
      const int tl = lane / 2, hf = lane % 2;
      float y[64];
      for (int q = 0; q < 8; q++) {
        const uint32_t w[4] = {kr[q].x, kr[q].y, kr[q].z, kr[q].w};
        for (int e = 0; e < 4; e++) {
          y[8 * q + 2 * e] = __half2float(__ushort_as_half(static_cast<unsigned short>(w[e] & 0xFFFFu)));
          y[8 * q + 2 * e + 1] = __half2float(__ushort_as_half(static_cast<unsigned short>(w[e] >> 16)));
        }
      }
      if (t0 + tl >= t_old) {  // the partner lane (same token) takes the same branch
        for (int hw = 1; hw < 64; hw <<= 1)
          for (int j = 0; j < 64; j += 2 * hw)
            for (int k = j; k < j + hw; k++) {
              const float a = y[k], c = y[k + hw];
              y[k] = a + c;
              y[k + hw] = a - c;
            }
        for (int k = 0; k < 64; k++) {
          const float o = __builtin_bit_cast(
              float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, y[k]), 0xB1, 0xF, 0xF, false));
          y[k] = hf == 0 ? y[k] + o : o - y[k];  // (channel c, c + 64) -> (sum, difference)
        }
        for (int k = 0; k < 64; k++) {
          float v = y[k] * kInvSqrt128;
          asm volatile("" : "+v"(v));  // round the product to fp32 first
          y[k] = __half2float(__float2half_rn(v));
        }
      }
      for (int k = 0; k < 64; k += 2)
        *reinterpret_cast<__half2*>(&kt[tl][64 * hf + k]) = __floats2half2_rn(y[k], y[k + 1]);
      __syncthreads();
      for (int i = 0; i < kG; i++) {
        const __half2 v = *reinterpret_cast<const __half2*>(&kt[i][2 * lane]);
        x0[i] = __low2float(v);
        x1[i] = __high2float(v);
      }
      __syncthreads();  // the key codes overwrite these bytes next
    } else {
      for (int i = 0; i < kG; i++) {
        x0[i] = __half2float(__ushort_as_half(static_cast<unsigned short>(ku[i] & 0xFFFFu)));
        x1[i] = __half2float(__ushort_as_half(static_cast<unsigned short>(ku[i] >> 16)));
      }
    }
    uint8_t c0[kG], c1[kG];
    const QuantOut r0 = quantize_regs<BITS>(x0, c0);
    const QuantOut r1 = quantize_regs<BITS>(x1, c1);
    for (int i = 0; i < kG; i++)
      *reinterpret_cast<uint16_t*>(&ck[i][2 * lane]) = uint16_t(c0[i]) | uint16_t(c1[i]) << 8;
    uint32_t* sz = reinterpret_cast<uint32_t*>(blk + 2 * CB);
    sz[lane] = uint32_t(__half_as_ushort(r0.s)) | uint32_t(__half_as_ushort(r1.s)) << 16;
    sz[kD / 2 + lane] = uint32_t(__half_as_ushort(r0.z)) | uint32_t(__half_as_ushort(r1.z)) << 16;
  }
  // Values.
  for (int k = 0; k < 2; k++) {
    const int i = 16 * k + lane / 4, j = lane % 4;
    float x[kG];
    for (int q = 0; q < 4; q++) {
      const uint4 u = vu[k][q];
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
      for (int e = 0; e < 4; e++) {
        x[8 * q + 2 * e] = __half2float(__ushort_as_half(static_cast<unsigned short>(w[e] & 0xFFFFu)));
        x[8 * q + 2 * e + 1] = __half2float(__ushort_as_half(static_cast<unsigned short>(w[e] >> 16)));
      }
    }
    uint8_t c[kG];
    const QuantOut r = quantize_regs<BITS>(x, c);
    uint32_t wds[kG / 4];
    for (int q = 0; q < kG / 4; q++)
      wds[q] = uint32_t(c[4 * q]) | uint32_t(c[4 * q + 1]) << 8 | uint32_t(c[4 * q + 2]) << 16 |
               uint32_t(c[4 * q + 3]) << 24;
    uint4* dst = reinterpret_cast<uint4*>(&cv[i][kG * j]);
    dst[0] = make_uint4(wds[0], wds[1], wds[2], wds[3]);
    dst[1] = make_uint4(wds[4], wds[5], wds[6], wds[7]);
    const int kb = (i % 16) / 4, sl = 4 * (i / 16) + i % 4;
    const int vi = (kb * 4 + j) * 8 + sl;
    vsz[0][vi] = r.s;
    vsz[1][vi] = r.z;
  }
  __syncthreads();

  // Packed words: key token i, channel d is slot d%8 of operand 2(d/32) + i/16 in
  // lane i%16 + 16((d%32)/8); value token i, channel d is slot 4(i/16) + i%4 of
  // operand d/16 in lane d%16 + 16((i%16)/4).
  uint32_t* kw = reinterpret_cast<uint32_t*>(blk);
  uint32_t* vw = reinterpret_cast<uint32_t*>(blk + CB);
  if constexpr (BITS == 3) {
    // Bits 0-1 of the codes: word (lane l, operand pair ohi), slot s of operand
    // 2 ohi + par at bit 8(s%4) + 4(s/4) + 2 par. Bit 2: word (lane l, operand
    // quad oq) at byte 1024 + 8 l + 4 oq, operand 4 oq + r at bit 8(s%4) + 4(s/4) + r.
    for (int w = lane; w < 256; w += 64) {
      uint32_t kword = 0, vword = 0;
      const int l = w / 4, ohi = w % 4;
      for (int par = 0; par < 2; par++) {
        const int o = 2 * ohi + par;
        for (int s2 = 0; s2 < 8; s2++) {
          const int bit = 8 * (s2 % 4) + 4 * (s2 / 4) + 2 * par;
          const int ki = 16 * (o % 2) + l % 16, kd = 32 * (o / 2) + 8 * (l / 16) + s2;
          const int vd = 16 * o + l % 16, vi = value_token(l / 16, s2);
          kword |= uint32_t(ck[ki][kd] & 3) << bit;
          vword |= uint32_t(cv[vi][vd] & 3) << bit;
        }
      }
      kw[w] = kword;
      vw[w] = vword;
    }
    for (int w = lane; w < 128; w += 64) {
      uint32_t kword = 0, vword = 0;
      const int l = w / 2, oq = w % 2;
      for (int r2 = 0; r2 < 4; r2++) {
        const int o = 4 * oq + r2;
        for (int s2 = 0; s2 < 8; s2++) {
          const int bit = 8 * (s2 % 4) + 4 * (s2 / 4) + r2;
          const int ki = 16 * (o % 2) + l % 16, kd = 32 * (o / 2) + 8 * (l / 16) + s2;
          const int vd = 16 * o + l % 16, vi = value_token(l / 16, s2);
          kword |= uint32_t(ck[ki][kd] >> 2) << bit;
          vword |= uint32_t(cv[vi][vd] >> 2) << bit;
        }
      }
      kw[256 + w] = kword;
      vw[256 + w] = vword;
    }
  }
  constexpr int NW = BITS == 3 ? 0 : CB / 4;
  for (int w = lane; w < NW; w += 64) {
    uint32_t kword = 0, vword = 0;
    if (BITS == 2) {
      const int l = w / 4, ohi = w % 4;
      for (int par = 0; par < 2; par++) {
        const int o = 2 * ohi + par;
        for (int s2 = 0; s2 < 8; s2++) {
          const int bit = 8 * (s2 / 2) + 4 * (s2 % 2) + 2 * par;
          const int ki = 16 * (o % 2) + l % 16, kd = 32 * (o / 2) + 8 * (l / 16) + s2;
          const int vd = 16 * o + l % 16, vi = value_token(l / 16, s2);
          kword |= uint32_t(ck[ki][kd]) << bit;
          vword |= uint32_t(cv[vi][vd]) << bit;
        }
      }
    } else {
      const int o = 4 * (w / 256) + w % 4, l = (w % 256) / 4;
      for (int s2 = 0; s2 < 8; s2++) {
        const int bit = 8 * (s2 % 4) + 4 * (s2 / 4);
        const int ki = 16 * (o % 2) + l % 16, kd = 32 * (o / 2) + 8 * (l / 16) + s2;
        const int vd = 16 * o + l % 16, vi = value_token(l / 16, s2);
        kword |= uint32_t(ck[ki][kd]) << bit;
        vword |= uint32_t(cv[vi][vd]) << bit;
      }
    }
    kw[w] = kword;
    vw[w] = vword;
  }
  uint32_t* vszw = reinterpret_cast<uint32_t*>(blk + 2 * CB + 512);
  const uint32_t* vszl = reinterpret_cast<const uint32_t*>(&vsz[0][0]);
  vszw[lane] = vszl[lane];
  vszw[64 + lane] = vszl[64 + lane];
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
  const SeqDesc sd = seq_record(seq, seq.dev, b);
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
  const GroupStore blocks = group_store(L, base);
  auto* rk = reinterpret_cast<const __half*>(base + L.ringk_off);
  auto* rv = reinterpret_cast<const __half*>(base + L.ringv_off);
  auto* kin = static_cast<const __half*>(k);
  auto* vin = static_cast<const __half*>(v);
#define KVQ_FLUSH(BITS, ROT)                                                                                  \
  hipLaunchKernelGGL((flush_wave_kernel<BITS, ROT>), grid, dim3(64), 0, stream, blocks, rk, rv, seq, kin, vin, L.Hkv, \
                     L.W, L.RS, L.sink, n_max)
  if (L.bits == 2) {
    if (rotate) KVQ_FLUSH(2, true);
    else KVQ_FLUSH(2, false);
  } else if (L.bits == 3) {
    if (rotate) KVQ_FLUSH(3, true);
    else KVQ_FLUSH(3, false);
  } else {
    if (rotate) KVQ_FLUSH(4, true);
    else KVQ_FLUSH(4, false);
  }
#undef KVQ_FLUSH
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
