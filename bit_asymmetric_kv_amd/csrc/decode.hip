// Decode-step attention read directly from the packed low-bit cache.
//
// Decode reads the whole cache at every step and is bound by memory traffic
// ("Read What Matters", the NOVA-KV and RDKV abstracts; "KV cache quantization:
// putting the bits in the cached vectors", the KIVI abstract on the compute core
// idling while the cache loads). Scores over the quantized groups and over the FP16
// residual are combined inside one attention computation (same page, full-text-skim
// notes on KIVI's grouped/residual split).
//
// Work split (flash-decoding style): one workgroup per (sequence split of whole
// groups, kv-head, sequence) plus one workgroup per (kv-head, sequence) for the FP16
// window; each writes partial (max, sum, unnormalized output) per query head, and a
// second kernel merges them.
//
// Inside a split each wave streams whole 32-token groups. Every group block is read
// from HBM once and serves all query heads of the kv-head:
//  * scores: an MFMA 16x16x32 f16 contraction over channels with the key codes as
//    A (converted exactly to f16 by the scaled fp4/fp8 conversions) and, as B, the
//    query multiplied by the group's per-channel key scale, split into fp16 high and
//    low parts (two columns per head, so the product keeps ~22 bits); the key
//    zero-points enter through q.z, computed once per group per head;
//  * values: an MFMA contraction over the group's tokens with the value codes as A
//    and, as B, the softmax weight times the per-token value scale (again high/low
//    columns); the value zero-points enter through sum_t p_t z_t per channel group.
#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>

#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kD = kHeadDim;
constexpr int kG = kGroup;
constexpr int kWaves = 4;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));

struct DecodeArgs {
  const uint8_t* blocks;
  const __half* ringk;
  const __half* ringv;
  const SeqDesc* seq;
  const __half* q;
  float* part;
  long long gcap;
  int Hkv, Hq, W, gps, nsplit, rotate;
  float scale_log2;
};

// 8 two-bit codes of one MFMA operand: `m` holds them in bits 0-1 and 4-5 of each
// byte (the other bits already masked off). As fp4 (e2m1) a nibble 00cc is c/2, so
// the scaled conversion with scale 2 returns c exactly.
__device__ inline half8 codes2_to_half8(uint32_t m) {
  half2v a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m, 2.0f, 0);
  half2v b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m, 2.0f, 1);
  half2v c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m, 2.0f, 2);
  half2v d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(m, 2.0f, 3);
  half8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// 8 four-bit codes in one word (slot s at bit 8*(s%4) + 4*(s/4)). A byte holding
// c in 0..15 reads as fp8 e4m3 c * 2^-9; the scaled conversion with 512 returns c.
__device__ inline half8 codes4_to_half8(uint32_t w) {
  uint32_t m0 = w & 0x0F0F0F0Fu, m1 = (w >> 4) & 0x0F0F0F0Fu;
  half2v a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(m0, 512.0f, false);
  half2v b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(m0, 512.0f, true);
  half2v c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(m1, 512.0f, false);
  half2v d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(m1, 512.0f, true);
  half8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// Operand o (0..7) of a lane's code section.
template <int BITS>
__device__ inline half8 code_operand(const uint4& w0, const uint4& w1, int o) {
  if constexpr (BITS == 2) {
    uint32_t w = (o / 2 == 0) ? w0.x : (o / 2 == 1) ? w0.y : (o / 2 == 2) ? w0.z : w0.w;
    return codes2_to_half8((w >> (2 * (o % 2))) & 0x33333333u);
  } else {
    const uint4& v = o < 4 ? w0 : w1;
    uint32_t w = (o % 4 == 0) ? v.x : (o % 4 == 1) ? v.y : (o % 4 == 2) ? v.z : v.w;
    return codes4_to_half8(w);
  }
}

// Value of the lane that holds the other (high or low) column of the same head.
// Columns are laid out as head h high at u = h, low at u = U - 1 - h (u = lane % U).
template <int U>
__device__ inline float partner(float x) {
  int xi = __builtin_bit_cast(int, x);
  int r;
  if constexpr (U == 2) r = __builtin_amdgcn_update_dpp(0, xi, 0xB1, 0xF, 0xF, false);        // quad_perm 1,0,3,2
  else if constexpr (U == 4) r = __builtin_amdgcn_update_dpp(0, xi, 0x1B, 0xF, 0xF, false);   // quad_perm 3,2,1,0
  else if constexpr (U == 8) r = __builtin_amdgcn_update_dpp(0, xi, 0x141, 0xF, 0xF, false);  // row_half_mirror
  else r = __builtin_amdgcn_update_dpp(0, xi, 0x140, 0xF, 0xF, false);                         // row_mirror
  return __builtin_bit_cast(float, r);
}

__device__ inline float wave_max_rows(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ inline float wave_sum_rows(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

__device__ inline half8 load_half8(const uint8_t* p) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(half8, u);
}

// Query preparation shared by all workgroups of one (kv-head, sequence): load the
// HG query rows, rotate (normalized Walsh-Hadamard, fp32) if the cache rotates,
// fold in softmax_scale * log2(e), and scale each head by a power of two 2^-e so
// that its largest entry is below 1 (keeps the fp16 high/low parts in range).
template <int HG>
__device__ void prepare_query(const DecodeArgs& a, int b, int h, float (*qf)[kD], float* expo) {
  for (int e = threadIdx.x; e < HG * kD; e += blockDim.x) {
    int hh = e / kD, d = e % kD;
    qf[hh][d] = __half2float(a.q[(size_t(b) * a.Hq + h * HG + hh) * kD + d]);
  }
  __syncthreads();
  if (a.rotate) {
    for (int hs = 1; hs < kD; hs <<= 1) {
      for (int p = threadIdx.x; p < HG * kD / 2; p += blockDim.x) {
        int hh = p / (kD / 2), j = p % (kD / 2);
        int ia = (j / hs) * (2 * hs) + (j % hs);
        float x = qf[hh][ia], y = qf[hh][ia + hs];
        qf[hh][ia] = x + y;
        qf[hh][ia + hs] = x - y;
      }
      __syncthreads();
    }
  }
  const float post = a.scale_log2 * (a.rotate ? 0x1.6a09e6p-4f : 1.0f);
  for (int e = threadIdx.x; e < HG * kD; e += blockDim.x) qf[e / kD][e % kD] *= post;
  __syncthreads();
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  for (int hh = wave; hh < HG; hh += kWaves) {
    float m = fmaxf(fabsf(qf[hh][lane]), fabsf(qf[hh][lane + 64]));
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    int ex = 0;
    if (m > 0.0f) frexpf(m, &ex);
    qf[hh][lane] = ldexpf(qf[hh][lane], -ex);
    qf[hh][lane + 64] = ldexpf(qf[hh][lane + 64], -ex);
    if (lane == 0) expo[hh] = ldexpf(1.0f, ex);
  }
  __syncthreads();
}

// Partial of one query head: running max m (log2 domain), sum l, output o[128].
__device__ inline float* partial_ptr(const DecodeArgs& a, int b, int hq, int split) {
  return a.part + ((size_t(b) * a.Hq + hq) * size_t(a.nsplit + 1) + split) * kPartialStride;
}

// Merge the per-wave partials held in shared memory (m, l, o per wave and head) and
// write the workgroup's partial.
template <int HG>
__device__ void merge_and_store(const DecodeArgs& a, int b, int h, int split, float (*wp)[HG][kPartialStride]) {
  __syncthreads();
  for (int idx = threadIdx.x; idx < HG * kPartialStride; idx += blockDim.x) {
    int hh = idx / kPartialStride, c = idx % kPartialStride;
    float M = -INFINITY;
    for (int w = 0; w < kWaves; w++) M = fmaxf(M, wp[w][hh][0]);
    float r;
    if (c == 0) {
      r = M;
    } else if (M == -INFINITY) {
      r = 0.0f;
    } else {
      r = 0.0f;
      for (int w = 0; w < kWaves; w++) {
        float mw = wp[w][hh][0];
        if (mw != -INFINITY) r += wp[w][hh][c] * exp2f(mw - M);
      }
    }
    partial_ptr(a, b, h * HG + hh, split)[c] = r;
  }
}

// Attention over the FP16 window [Q, T) of one (kv-head, sequence), in chunks of
// 256 tokens with a running max; the result goes to wave 0's slot of `wp`.
template <int HG>
__device__ void tail_attention(const DecodeArgs& a, int b, int h, int T, int Q, float (*qf)[kD],
                               const float* expo, float (*ts)[256], float (*wp)[HG][kPartialStride]) {
  constexpr int NOUT = (HG * kD + 255) / 256;
  __shared__ float m_s[HG], l_s[HG], alpha_s[HG];
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  const size_t bh = size_t(b) * a.Hkv + h;
  if (tid < HG) {
    m_s[tid] = -INFINITY;
    l_s[tid] = 0.0f;
  }
  float o[NOUT];
  for (int r = 0; r < NOUT; r++) o[r] = 0.0f;
  __syncthreads();
  for (int c0 = Q; c0 < T; c0 += 256) {
    const int cnt = min(256, T - c0);
    if (tid < cnt) {
      const uint8_t* krow = reinterpret_cast<const uint8_t*>(a.ringk + (bh * a.W + size_t((c0 + tid) % a.W)) * kD);
      float acc[HG];
      for (int hh = 0; hh < HG; hh++) acc[hh] = 0.0f;
      for (int d8 = 0; d8 < kD / 8; d8++) {
        half8 kv = load_half8(krow + 16 * d8);
        for (int s = 0; s < 8; s++)
          for (int hh = 0; hh < HG; hh++) acc[hh] += qf[hh][8 * d8 + s] * float(kv[s]);
      }
      for (int hh = 0; hh < HG; hh++) ts[hh][tid] = acc[hh] * expo[hh];
    } else {
      for (int hh = 0; hh < HG; hh++) ts[hh][tid] = -INFINITY;
    }
    __syncthreads();
    for (int hh = wave; hh < HG; hh += kWaves) {
      float m = -INFINITY;
      for (int t = lane; t < 256; t += 64) m = fmaxf(m, ts[hh][t]);
      for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
      const float m_old = m_s[hh];
      const float m_new = fmaxf(m_old, m);
      float sum = 0.0f;
      for (int t = lane; t < 256; t += 64) {
        float p = t < cnt ? exp2f(ts[hh][t] - m_new) : 0.0f;
        ts[hh][t] = p;
        sum += p;
      }
      for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
      if (lane == 0) {
        const float alpha = m_old == -INFINITY ? 0.0f : exp2f(m_old - m_new);
        alpha_s[hh] = alpha;
        l_s[hh] = l_s[hh] * alpha + sum;
        m_s[hh] = m_new;
      }
    }
    __syncthreads();
    for (int r = 0; r < NOUT; r++) {
      const int idx = tid + 256 * r;
      if (idx < HG * kD) {
        const int hh = idx / kD, d = idx % kD;
        float acc = o[r] * alpha_s[hh];
        for (int t = 0; t < cnt; t++)
          acc += ts[hh][t] * __half2float(a.ringv[(bh * a.W + size_t((c0 + t) % a.W)) * kD + d]);
        o[r] = acc;
      }
    }
    __syncthreads();
  }
  for (int r = 0; r < NOUT; r++) {
    const int idx = tid + 256 * r;
    if (idx < HG * kD) wp[0][idx / kD][2 + idx % kD] = o[r];
  }
  if (tid < HG) {
    wp[0][tid][0] = m_s[tid];
    wp[0][tid][1] = l_s[tid];
    for (int w = 1; w < kWaves; w++) wp[w][tid][0] = -INFINITY;
  }
}

template <int BITS, int HG>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
  constexpr int U = 2 * HG;                   // useful MFMA columns: high and low part per head
  constexpr int REP = 16 / U;                 // replicas of those columns across the 16 columns
  constexpr int NJ = REP >= 4 ? 1 : 4 / REP;  // value channel groups handled per lane
  constexpr int CB = kG * kD * BITS / 8;      // bytes of one code section
  constexpr int GB = 2 * CB + 1024;           // bytes of one group block
  constexpr int ITEMS = (HG + 3) / 4;         // key-side operand items per lane

  __shared__ float qf[HG][kD];
  __shared__ float expo[HG];
  __shared__ union {
    half8 bk[kWaves][4][U][4];  // key-side B operands per wave: [kc][column][k-block]
    float ts[HG][256];          // FP16-window scores
  } sh;
  __shared__ float wp[kWaves][HG][kPartialStride];

  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const SeqDesc sd = a.seq[b];
  const int T = sd.t_old + sd.n_new, Q = sd.q_new;
  const int ng = Q / kG;

  prepare_query<HG>(a, b, h, qf, expo);

  if (split == a.nsplit) {
    tail_attention<HG>(a, b, h, T, Q, qf, expo, sh.ts, wp);
    merge_and_store<HG>(a, b, h, split, wp);
    return;
  }

  const int g0 = split * a.gps;
  const int g1 = min(ng, g0 + a.gps);
  const int len = max(0, g1 - g0);
  const int per = (len + kWaves - 1) / kWaves;
  const int wg0 = g0 + wave * per;
  const int wg1 = min(g1, wg0 + per);

  // MFMA lane roles: column n = lane % 16, k-block / row block kb = lane / 16.
  const int n = lane % 16, kb = lane / 16;
  const int u = n % U;
  const bool ishi = u < HG;
  const int hd = ishi ? u : U - 1 - u;  // query head of this lane's column
  const int rho = n / U;                // replica index of this column
  const int jbase = (rho % (4 / NJ)) * NJ;

  // Key-side operand preparation: channel block cb (8 channels), heads hh0 + 4 * it.
  const int cb = lane % 16, hh0 = lane / 16;
  float qreg[ITEMS][8];
  for (int it = 0; it < ITEMS; it++)
    for (int s = 0; s < 8; s++) {
      const int hh = hh0 + 4 * it;
      qreg[it][s] = hh < HG ? qf[hh][8 * cb + s] : 0.0f;
    }
  const float ex = expo[hd];

  float4v oacc[8];
  for (int t = 0; t < 8; t++) oacc[t] = float4v{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;
  float zacc[NJ];
  for (int jr = 0; jr < NJ; jr++) zacc[jr] = 0.0f;

  const uint8_t* base = a.blocks + (size_t(b) * a.Hkv + h) * size_t(a.gcap) * GB;
  for (int g = wg0; g < wg1; g++) {
    const uint8_t* blk = base + size_t(g) * GB;
    const uint4 kc0 = *reinterpret_cast<const uint4*>(blk + 16 * lane);
    const uint4 kc1 = BITS == 4 ? *reinterpret_cast<const uint4*>(blk + 1024 + 16 * lane) : kc0;
    const uint4 vc0 = *reinterpret_cast<const uint4*>(blk + CB + 16 * lane);
    const uint4 vc1 = BITS == 4 ? *reinterpret_cast<const uint4*>(blk + CB + 1024 + 16 * lane) : vc0;
    const half8 ks8 = load_half8(blk + 2 * CB + 16 * cb);
    const half8 kz8 = load_half8(blk + 2 * CB + 256 + 16 * cb);
    half8 vs8[NJ], vz8[NJ];
    for (int jr = 0; jr < NJ; jr++) {
      const int j = jbase + jr;
      vs8[jr] = load_half8(blk + 2 * CB + 512 + 16 * (kb * 4 + j));
      vz8[jr] = load_half8(blk + 2 * CB + 768 + 16 * (kb * 4 + j));
    }

    // q' = q * s_key (per channel) as fp16 high + low parts; q.z_key per head.
    float qz[ITEMS];
    for (int it = 0; it < ITEMS; it++) {
      const int hh = hh0 + 4 * it;
      half8 hi, lo;
      float z = 0.0f;
      for (int s = 0; s < 8; s++) {
        const float qp = qreg[it][s] * float(ks8[s]);
        const _Float16 hv = _Float16(qp);
        hi[s] = hv;
        lo[s] = _Float16(qp - float(hv));
        z += qreg[it][s] * float(kz8[s]);
      }
      for (int off = 1; off < 16; off <<= 1) z += __shfl_xor(z, off);
      qz[it] = z;
      if (hh < HG) {
        sh.bk[wave][cb / 4][hh][cb % 4] = hi;
        sh.bk[wave][cb / 4][U - 1 - hh][cb % 4] = lo;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    float qzc;
    if constexpr (ITEMS == 1) {
      qzc = __shfl(qz[0], 16 * (hd % 4));
    } else {
      const float q0 = __shfl(qz[0], 16 * (hd % 4));
      const float q1 = __shfl(qz[1], 16 * (hd % 4));
      qzc = hd >= 4 ? q1 : q0;
    }
    const float init = ishi ? qzc : 0.0f;

    // Scores of the group's 32 tokens: rows 4*kb + i of tiles 0 and 1.
    float4v s0 = {init, init, init, init}, s1 = s0;
    for (int kc = 0; kc < 4; kc++) {
      const half8 bk = sh.bk[wave][kc][u][kb];
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(code_operand<BITS>(kc0, kc1, 2 * kc), bk, s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(code_operand<BITS>(kc0, kc1, 2 * kc + 1), bk, s1, 0, 0, 0);
    }
    float sc[8];
    for (int i = 0; i < 4; i++) {
      sc[i] = (s0[i] + partner<U>(s0[i])) * ex;
      sc[4 + i] = (s1[i] + partner<U>(s1[i])) * ex;
    }

    // Online softmax (log2 domain), shared by every lane of the head.
    float mloc = sc[0];
    for (int i = 1; i < 8; i++) mloc = fmaxf(mloc, sc[i]);
    mloc = wave_max_rows(mloc);
    const float m_new = fmaxf(m_run, mloc);
    if (__ballot(m_new > m_run)) {
      const float alpha = m_run == -INFINITY ? 0.0f : exp2f(m_run - m_new);
      for (int t = 0; t < 8; t++) oacc[t] *= alpha;
      l_run *= alpha;
      for (int jr = 0; jr < NJ; jr++) zacc[jr] *= alpha;
      m_run = m_new;
    }
    float p[8];
    for (int i = 0; i < 8; i++) {
      p[i] = __builtin_amdgcn_exp2f(sc[i] - m_run);
      l_run += p[i];
    }

    // Value side: B = p * s_value (high or low part by column), plus sum p * z.
    half8 bv[NJ];
    for (int jr = 0; jr < NJ; jr++) {
      float z = zacc[jr];
      for (int s = 0; s < 8; s++) {
        const float pp = p[s] * float(vs8[jr][s]);
        const _Float16 hv = _Float16(pp);
        bv[jr][s] = ishi ? hv : _Float16(pp - float(hv));
        z += p[s] * float(vz8[jr][s]);
      }
      zacc[jr] = z;
    }
    for (int t = 0; t < 8; t++)
      oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(code_operand<BITS>(vc0, vc1, t), bv[(t / 2) % NJ], oacc[t],
                                                       0, 0, 0);
  }

  // Wave partial: sums over the four row blocks, high + low columns.
  const float l_tot = wave_sum_rows(l_run);
  float zs[NJ];
  for (int jr = 0; jr < NJ; jr++) zs[jr] = wave_sum_rows(zacc[jr]);
  if (kb == 0 && ishi && rho == 0) {
    wp[wave][hd][0] = m_run;
    wp[wave][hd][1] = l_tot;
  }
  for (int t = 0; t < 8; t++) {
    const int valid_rho = (t / 2) / NJ;
    for (int i = 0; i < 4; i++) {
      const float v = oacc[t][i] + partner<U>(oacc[t][i]);
      if (ishi && rho == valid_rho) wp[wave][hd][2 + 16 * t + 4 * kb + i] = v + zs[(t / 2) % NJ];
    }
  }
  merge_and_store<HG>(a, b, h, split, wp);
}

// out[b][hq] = sum_i o_i 2^(m_i - M) / sum_i l_i 2^(m_i - M) over the partials of
// one (sequence, query head). 512 threads: the partials' weights are computed once
// into shared memory, then 4 slices of 128 threads (one per channel) sum strided
// subsets of the partials and are added at the end.
constexpr int kCombineThreads = 512;
constexpr int kCombineMaxParts = kMaxSplits + 1;

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const float* __restrict__ part,
                                                                  float* __restrict__ out, int Hq, int nparts) {
  __shared__ float wgt[kCombineMaxParts];
  __shared__ float red[kCombineThreads / 64];
  __shared__ float osum[kCombineThreads / kD][kD];
  const int hq = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64;
  const float* p = part + (size_t(b) * Hq + hq) * size_t(nparts) * kPartialStride;

  float m = -INFINITY;
  for (int i = tid; i < nparts; i += kCombineThreads) m = fmaxf(m, p[size_t(i) * kPartialStride]);
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  float M = red[0];
  for (int w = 1; w < kCombineThreads / 64; w++) M = fmaxf(M, red[w]);
  __syncthreads();

  float l = 0.0f;
  for (int i = tid; i < nparts; i += kCombineThreads) {
    const float mi = p[size_t(i) * kPartialStride];
    const float wi = mi == -INFINITY ? 0.0f : exp2f(mi - M);
    wgt[i] = wi;
    l += wi * p[size_t(i) * kPartialStride + 1];
  }
  for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o);
  if (lane == 0) red[wave] = l;
  __syncthreads();
  float L = 0.0f;
  for (int w = 0; w < kCombineThreads / 64; w++) L += red[w];

  const int d = tid % kD, slice = tid / kD;
  constexpr int kSlices = kCombineThreads / kD;
  float o = 0.0f;
  for (int i = slice; i < nparts; i += kSlices) {
    const float wi = wgt[i];
    if (wi != 0.0f) o += wi * p[size_t(i) * kPartialStride + 2 + d];
  }
  osum[slice][d] = o;
  __syncthreads();
  if (slice == 0) {
    float acc = 0.0f;
    for (int s2 = 0; s2 < kSlices; s2++) acc += osum[s2][d];
    out[(size_t(b) * Hq + hq) * kD + d] = acc / L;
  }
}

template <int BITS, int HG>
hipError_t launch_split(const DecodeArgs& a, int B, hipStream_t stream) {
  hipLaunchKernelGGL((decode_split_kernel<BITS, HG>), dim3(a.nsplit + 1, a.Hkv, B), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const Layout& L, uint8_t* base, const SeqDesc* seq, const void* q, float* out,
                         int32_t groups_per_split, int32_t nsplit, float scale_log2, int rotate, hipStream_t stream,
                         hipEvent_t prof_start, hipEvent_t prof_stop) {
  DecodeArgs a;
  a.blocks = base + L.blocks_off;
  a.ringk = reinterpret_cast<const __half*>(base + L.ringk_off);
  a.ringv = reinterpret_cast<const __half*>(base + L.ringv_off);
  a.seq = seq;
  a.q = static_cast<const __half*>(q);
  a.part = reinterpret_cast<float*>(base + L.part_off);
  a.gcap = L.gcap;
  a.Hkv = L.Hkv;
  a.Hq = L.Hq;
  a.W = L.W;
  a.gps = groups_per_split;
  a.nsplit = nsplit;
  a.rotate = rotate;
  a.scale_log2 = scale_log2;
  const int hg = L.Hq / L.Hkv;
  hipError_t e;
  if (prof_start && hipEventRecord(prof_start, stream) != hipSuccess) return hipGetLastError();
  if (L.bits == 2) {
    e = hg == 1 ? launch_split<2, 1>(a, L.B, stream)
        : hg == 2 ? launch_split<2, 2>(a, L.B, stream)
        : hg == 4 ? launch_split<2, 4>(a, L.B, stream)
                  : launch_split<2, 8>(a, L.B, stream);
  } else {
    e = hg == 1 ? launch_split<4, 1>(a, L.B, stream)
        : hg == 2 ? launch_split<4, 2>(a, L.B, stream)
        : hg == 4 ? launch_split<4, 4>(a, L.B, stream)
                  : launch_split<4, 8>(a, L.B, stream);
  }
  if (e != hipSuccess) return e;
  if (prof_stop && hipEventRecord(prof_stop, stream) != hipSuccess) return hipGetLastError();
  hipLaunchKernelGGL(combine_kernel, dim3(L.Hq, L.B), dim3(kCombineThreads), 0, stream, a.part, out, L.Hq, nsplit + 1);
  return hipGetLastError();
}

}  // namespace kvq
