// gfx950 kernels of the TARA attention library.
//
// What is computed ("TARA: Native Temporal Alignment for MiniMax H3
// References", section "The temporal rule"; "BFS H3 Reference Attention
// Binding (Experimental)", section "The exact rule"): one softmax over all keys
// of a packed sequence with logit
//     (Q.K) * scale - [target q, guide k] min(strength*(max(|tq-tk|-window,0)/falloff)^2, cap)
//                   + [target q, picture k, binding] m_q * ln(gain_pic)
// returning O and the natural-log LSE per query row.
//
// Kernels
//   meta_kernel        per-token encodings + per-64-key tile summaries  (O(N))
//   vtranspose_kernel  V [B,H,N,D] -> V^T [B*H][D][npad], keys contiguous (HBM-bound)
//   attn_bf16_kernel   the fused pass: bf16 MFMA S^T = K Q^T, bias, online
//                      softmax, MFMA O^T += V^T P^T, one workgroup per block
//                      of query rows of one (batch, head), streaming all key
//                      tiles of its key range through LDS
//   attn_f32_kernel    fp32 inputs: same arithmetic with FMA (correctness path)
//   merge_kernel       exact LSE merge of per-partition (O_p, LSE_p)
//
// Layout facts the bf16 kernel relies on (v_mfma_f32_32x32x16_bf16, wave64):
//   A operand: lane l holds row (l % 32), 8 consecutive k of k-half (l / 32)
//   B operand: lane l holds column (l % 32), the same 8 k of k-half (l / 32)
//   C/D:       lane l, register r holds row 8*(r/4) + 4*(l/32) + (r%4),
//              column l % 32.
// Computing S^T (keys x queries) puts one query per lane (column l % 32); each
// lane then owns 16 keys of a 32-key block and row statistics need only one
// exchange between lanes l and l^32. Loading K rows in the permuted order
// perm(r) (bits 2 and 3 swapped) makes the 16 keys a lane owns two runs of 8
// consecutive keys, so P^T feeds the P.V product straight from registers and
// V^T fragments are single 16-byte LDS reads.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "tara_internal.h"

namespace tara {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.6931471805599453f;
// Lazy rescaling threshold (log2 units): the running max used for the
// exponent is only moved when a row's max grows by more than this, so
// unnormalised probabilities stay <= 2^8.
constexpr float kRescaleTau = 8.0f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine a value with the one held by lane l ^ 32 (max or sum).
__device__ __forceinline__ float xor32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// Workgroups are dispatched round-robin over the 8 XCDs; map the dispatch id
// to a logical id so that each XCD works through a contiguous range of
// (batch*head, query block): the blocks resident on one XCD then share one
// head's K/V stream in that XCD's L2.
__device__ __forceinline__ int xcd_remap(int pid, int total) {
  constexpr int X = 8;
  const int per = (total + X - 1) / X;
  const int tall = total - (per - 1) * X;
  const int x = pid % X, s = pid / X;
  return x < tall ? x * per + s : tall * per + (x - tall) * (per - 1) + s;
}

// ------------------------------------------------------------------ metadata
// One 64-thread workgroup per (key tile, batch element).
__global__ __launch_bounds__(64) void meta_kernel(MetaArgs a) {
  const int b = blockIdx.y;
  const int n = blockIdx.x * kBlockK + threadIdx.x;
  const bool valid = n < a.N;
  const int64_t mi = (int64_t)b * a.N + n;
  int seg = valid ? (int)a.seg[mi] : 3;
  const float t = valid ? a.time[mi] : 0.0f;
  const bool tfinite = valid && isfinite(t);
  const float nanv = __builtin_nanf("");

  // query side (n < N only)
  if (valid) {
    const bool tgt = seg == 0;
    a.tq[mi] = (tgt && a.bias_active && tfinite) ? t : nanv;
    float m = 0.0f;
    if (tgt && a.binding_active) m = a.mask ? a.mask[mi] : 1.0f;
    a.mq[mi] = m;
  }
  // key side (n < npad)
  const bool isg = valid && seg == 1 && a.bias_active && tfinite;
  const float tk = isg ? t : nanv;
  float kbv = 0.0f;
  if (valid && seg == 2 && a.binding_active) {
    const int id = a.pic[mi];
    if (id >= 0 && id < a.num_pictures) kbv = a.lg2gain[id];
  }
  const int64_t ki = (int64_t)b * a.npad + n;
  a.tk[ki] = tk;
  a.kb[ki] = kbv;

  // tile summary
  const bool isp = kbv != 0.0f;
  const bool all_plain = !wave_any(isg || isp);
  const bool all_guide = !wave_any(!isg);
  const float kb0 = __shfl(kbv, 0);
  const bool all_pic = !wave_any(!isp || kbv != kb0);
  float lo = isg ? tk : INFINITY, hi = isg ? tk : -INFINITY;
  for (int off = 32; off >= 1; off >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, off));
    hi = fmaxf(hi, __shfl_xor(hi, off));
  }
  if (threadIdx.x == 0) {
    KeyTileSummary s;
    s.kind = all_plain ? KT_PLAIN : all_guide ? KT_GUIDE : all_pic ? KT_PICTURE : KT_MIXED;
    s.lo = lo;
    s.hi = hi;
    s.bias = all_pic ? kb0 : 0.0f;
    a.ksum[(int64_t)b * a.nkt + blockIdx.x] = s;
  }
}

hipError_t launch_meta(const MetaArgs& a, hipStream_t s) {
  dim3 grid(a.npad / kBlockK, a.B);
  hipLaunchKernelGGL(meta_kernel, grid, dim3(64), 0, s, a);
  return hipGetLastError();
}

// ------------------------------------------------------------- V transpose
// 64 keys x 64 dims per workgroup through LDS; keys >= N are written as 0.
__global__ __launch_bounds__(256) void vtranspose_kernel(const __bf16* __restrict__ v, int64_t sb,
                                                         int64_t sh, int64_t sn,
                                                         __bf16* __restrict__ vt, int H, int N,
                                                         int npad, int D) {
  __shared__ uint16_t tile[64][66];
  const int n0 = blockIdx.x * 64, d0 = blockIdx.y * 64, bh = blockIdx.z;
  const int b = bh / H, h = bh % H;
  const uint16_t* src = reinterpret_cast<const uint16_t*>(v) + b * sb + h * sh;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + i * 256;
    const int r = c >> 3, c8 = c & 7;
    const int n = n0 + r;
    uint4 x = make_uint4(0, 0, 0, 0);
    if (n < N) x = *reinterpret_cast<const uint4*>(src + (int64_t)n * sn + d0 + c8 * 8);
    const uint16_t* e = reinterpret_cast<const uint16_t*>(&x);
#pragma unroll
    for (int j = 0; j < 8; ++j) tile[r][c8 * 8 + j] = e[j];
  }
  __syncthreads();
  uint16_t* dst = reinterpret_cast<uint16_t*>(vt) + (int64_t)bh * D * npad;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + i * 256;
    const int dr = c >> 3, c8 = c & 7;
    uint4 x;
    uint16_t* e = reinterpret_cast<uint16_t*>(&x);
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = tile[c8 * 8 + j][dr];
    *reinterpret_cast<uint4*>(dst + (int64_t)(d0 + dr) * npad + n0 + c8 * 8) = x;
  }
}

hipError_t launch_vtranspose(const __bf16* v, int64_t sb, int64_t sh, int64_t sn, __bf16* vt,
                             int B, int H, int N, int npad, int D, hipStream_t s) {
  dim3 grid(npad / 64, D / 64, B * H);
  hipLaunchKernelGGL(vtranspose_kernel, grid, dim3(256), 0, s, v, sb, sh, sn, vt, H, N, npad, D);
  return hipGetLastError();
}

// --------------------------------------------------------- bf16 MFMA kernel
constexpr int kWaves = 4;                 // waves per workgroup
constexpr int kQW = 32;                   // query rows per wave
constexpr int kBQ = kWaves * kQW;         // query rows per workgroup

// Key row held by S^T output row `r` of a 32-key block: bits 2 and 3 swapped.
__device__ __forceinline__ int perm32(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Global -> registers part of staging one key tile: K rows [kt*64, kt*64+64)
// (rows past N clamped to N-1; those keys are masked later) and the matching
// 64 key columns of V^T (zero-padded to npad).
template <int D, int NT, int KCH, int VCH>
__device__ __forceinline__ void load_kv_tile(u32x4 (&pk)[KCH], u32x4 (&pv)[VCH], const __bf16* kg,
                                             int64_t k_sn, const __bf16* vg, int npad, int kt, int N,
                                             int tid) {
#pragma unroll
  for (int i = 0; i < KCH; ++i) {
    const int c = tid + i * NT;
    const int r = c / (D / 8), c8 = c % (D / 8);
    const int n = min(kt * kBlockK + r, N - 1);
    pk[i] = *reinterpret_cast<const u32x4*>(kg + (int64_t)n * k_sn + c8 * 8);
  }
#pragma unroll
  for (int i = 0; i < VCH; ++i) {
    const int c = tid + i * NT;
    const int d = c / (kBlockK / 8), c8 = c % (kBlockK / 8);
    pv[i] = *reinterpret_cast<const u32x4*>(vg + (int64_t)d * npad + kt * kBlockK + c8 * 8);
  }
}

// Registers -> LDS part: K tile as [64][KROW], V^T tile as [D][VROW].
template <int D, int NT, int KCH, int VCH, int KROW, int VROW>
__device__ __forceinline__ void store_kv_tile(const u32x4 (&pk)[KCH], const u32x4 (&pv)[VCH], __bf16* ks,
                                              __bf16* vs, int tid) {
#pragma unroll
  for (int i = 0; i < KCH; ++i) {
    const int c = tid + i * NT;
    const int r = c / (D / 8), c8 = c % (D / 8);
    *reinterpret_cast<u32x4*>(ks + r * KROW + c8 * 8) = pk[i];
  }
#pragma unroll
  for (int i = 0; i < VCH; ++i) {
    const int c = tid + i * NT;
    const int d = c / (kBlockK / 8), c8 = c % (kBlockK / 8);
    *reinterpret_cast<u32x4*>(vs + d * VROW + c8 * 8) = pv[i];
  }
}

template <int D, bool PART>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void attn_bf16_kernel(AttnArgs a) {
  constexpr int NT = kWaves * 64;
  constexpr int KROW = D + 8;              // padded LDS pitch of a K row (elements)
  constexpr int VROW = kBlockK + 8;        // padded LDS pitch of a V^T row (elements)
  constexpr int KTILE = kBlockK * KROW;
  constexpr int VTILE = D * VROW;
  constexpr int STAGE = KTILE + VTILE;
  constexpr int KCH = kBlockK * D / 8 / NT;   // 16-byte chunks per thread, K tile
  constexpr int VCH = D * kBlockK / 8 / NT;   // 16-byte chunks per thread, V^T tile
  constexpr int NKK = D / 16;                 // MFMA k-steps over the head dim
  constexpr int NDB = D / 32;                 // 32-row blocks of O^T
  static_assert(KCH * NT * 8 == kBlockK * D && VCH * NT * 8 == kBlockK * D, "tile split");
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * STAGE];

  const int part = PART ? blockIdx.y : 0;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = L / a.nqb, qblk = L % a.nqb;
  const int b = bh / a.H, h = bh % a.H;
  const int N = a.N;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lq = lane & 31, hh = lane >> 5;
  const int qrow = qblk * kBQ + wave * kQW + lq;
  const bool qvalid = qrow < N;
  const int qr = qvalid ? qrow : N - 1;

  const __bf16* qp = static_cast<const __bf16*>(a.q) + b * a.q_sb + h * a.q_sh + (int64_t)qr * a.q_sn;
  bf16x8 qf[NKK];
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qp + kk * 16 + hh * 8);
  const float tq = a.tq[(int64_t)b * N + qr];
  const float mq = a.mq[(int64_t)b * N + qr];
  const bool qbiased = tq == tq;

  const int k0 = a.kr[part], k1 = a.kr[part + 1];
  // an empty key range visits no tile (a range inside one tile would
  // otherwise mask every key of it)
  const int kt0 = k0 / kBlockK, kt1 = k1 > k0 ? (k1 + kBlockK - 1) / kBlockK : kt0;

  f32x16 o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o[i] = f32x16{};
  float m_used = -INFINITY, lsum = 0.0f;

  const __bf16* kg = static_cast<const __bf16*>(a.k) + b * a.k_sb + h * a.k_sh;
  const __bf16* vg = a.vt + (int64_t)bh * D * a.npad;
  const float* tkb = a.tk + (int64_t)b * a.npad;
  const float* kbb = a.kb + (int64_t)b * a.npad;
  const KeyTileSummary* ks_b = a.ksum + (int64_t)b * a.nkt;

  u32x4 pk[KCH], pv[VCH];
  if (kt0 < kt1) {
    load_kv_tile<D, NT, KCH, VCH>(pk, pv, kg, a.k_sn, vg, a.npad, kt0, N, tid);
    store_kv_tile<D, NT, KCH, VCH, KROW, VROW>(pk, pv, smem, smem + KTILE, tid);
    __syncthreads();
  }
  const int krow_lane = perm32(lq);

  for (int kt = kt0, it = 0; kt < kt1; ++kt, ++it) {
    const int buf = it & 1;
    const bool more = kt + 1 < kt1;
    if (more) load_kv_tile<D, NT, KCH, VCH>(pk, pv, kg, a.k_sn, vg, a.npad, kt + 1, N, tid);
    const __bf16* ks = smem + buf * STAGE;
    const __bf16* vs = ks + KTILE;

    // S^T = K Q^T for the two 32-key blocks of the tile
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const __bf16* kr = ks + (kb * 32 + krow_lane) * KROW + hh * 8;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *reinterpret_cast<const bf16x8*>(kr + kk * 16), qf[kk], s[kb], 0, 0, 0);
    }

    // bias class of this (wave, key tile)
    const int kbase = kt * kBlockK;
    const bool partial = kbase < k0 || kbase + kBlockK > k1;
    float brow = 0.0f;
    bool elem = partial;
    if (!partial) {
      const KeyTileSummary sm = ks_b[kt];
      bool lane_elem = false;
      if (sm.kind == KT_GUIDE) {
        if (qbiased) {
          const float dlo = sm.lo - tq, dhi = tq - sm.hi;
          const float dmin = fmaxf(fmaxf(dlo, dhi), 0.0f);
          const float dmax = fmaxf(-dlo, -dhi);
          if (dmin >= a.dsat) brow = -a.cap2;
          else if (!(dmax <= a.window)) lane_elem = true;
        }
      } else if (sm.kind == KT_PICTURE) {
        brow = mq * sm.bias;
      } else if (sm.kind == KT_MIXED) {
        lane_elem = true;
      }
      elem = wave_any(lane_elem);
    }
    float cc = a.c;
    if (elem) {
      // per-element bias; keys outside [k0, k1) get -inf
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const int kx = kbase + kb * 32 + c2 * 16 + hh * 8;
          const f32x4 t0 = *reinterpret_cast<const f32x4*>(tkb + kx);
          const f32x4 t1 = *reinterpret_cast<const f32x4*>(tkb + kx + 4);
          const f32x4 g0 = *reinterpret_cast<const f32x4*>(kbb + kx);
          const f32x4 g1 = *reinterpret_cast<const f32x4*>(kbb + kx + 4);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float tk = e < 4 ? t0[e] : t1[e - 4];
            const float gk = e < 4 ? g0[e] : g1[e - 4];
            const float dd = fmaxf(fmaf(fabsf(tq - tk), a.sigma, -a.w), 0.0f);   // NaN time -> 0
            const float pen = fminf(dd * dd, a.cap2);
            float x = fmaf(s[kb][c2 * 8 + e], a.c, fmaf(mq, gk, -pen));
            if (partial && (kx + e < k0 || kx + e >= k1)) x = -INFINITY;
            s[kb][c2 * 8 + e] = x;
          }
        }
      }
      cc = 1.0f;
    }

    // online softmax (exp2 domain), lazily rescaled
    float mx = s[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = xor32_max(mx);
    const float mt = fmaf(mx, cc, brow);
    const bool grow = mt > m_used + kRescaleTau;
    if (wave_any(grow)) {
      const float mn = grow ? mt : m_used;
      const float alpha = fast_exp2(m_used - mn);
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < NDB; ++i) o[i] *= alpha;
      m_used = mn;
    }
    const float off = brow - m_used;
    bf16x8 pf[2][2];
    float tsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = fast_exp2(fmaf(s[kb][c2 * 8 + e], cc, off));
          tsum += p;
          pf[kb][c2][e] = (__bf16)p;
        }
    lsum += tsum;

    // O^T += V^T P^T
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const __bf16* vr = vs + lq * VROW + kb * 32 + c2 * 16 + hh * 8;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              *reinterpret_cast<const bf16x8*>(vr + db * 32 * VROW), pf[kb][c2], o[db], 0, 0, 0);
      }

    if (more)
      store_kv_tile<D, NT, KCH, VCH, KROW, VROW>(pk, pv, smem + (buf ^ 1) * STAGE,
                                                 smem + (buf ^ 1) * STAGE + KTILE, tid);
    __syncthreads();
  }

  // epilogue
  const float ltot = xor32_sum(lsum);
  if (!qvalid) return;
  if (kt0 >= kt1) {
    if (!PART) return;   // fused calls always have N >= 1 keys
    // empty partition: contributes nothing to the merge
    float* op = a.opart + ((((int64_t)part * a.B + b) * a.H + h) * N + qrow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<f32x4*>(op + db * 32 + j * 8 + hh * 4) = f32x4{};
    if (hh == 0) a.lsepart[(((int64_t)part * a.B + b) * a.H + h) * N + qrow] = -INFINITY;
    return;
  }
  const float inv = 1.0f / ltot;
  const float lse = (m_used + __log2f(ltot)) * kLn2;
  if (PART) {
    float* op = a.opart + ((((int64_t)part * a.B + b) * a.H + h) * N + qrow) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = o[db][j * 4 + i] * inv;
        *reinterpret_cast<f32x4*>(op + db * 32 + j * 8 + hh * 4) = x;
      }
    if (hh == 0) a.lsepart[(((int64_t)part * a.B + b) * a.H + h) * N + qrow] = lse;
  } else {
    __bf16* op = static_cast<__bf16*>(a.o) + b * a.o_sb + h * a.o_sh + (int64_t)qrow * a.o_sn;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = (__bf16)(o[db][j * 4 + i] * inv);
        *reinterpret_cast<bf16x4*>(op + db * 32 + j * 8 + hh * 4) = x;
      }
    if (hh == 0) a.lse[((int64_t)b * a.H + h) * N + qrow] = lse;
  }
}

int attn_bf16_block_q(int) { return kBQ; }

int attn_bf16_grid(const AttnArgs& a) { return a.nqb * a.B * a.H; }

hipError_t launch_attn_bf16(const AttnArgs& a, int D, bool partitioned, hipStream_t s) {
  dim3 grid(attn_bf16_grid(a), partitioned ? a.nparts : 1);
  dim3 block(kWaves * 64);
  if (D == 128) {
    if (partitioned) hipLaunchKernelGGL((attn_bf16_kernel<128, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((attn_bf16_kernel<128, false>), grid, block, 0, s, a);
  } else {
    if (partitioned) hipLaunchKernelGGL((attn_bf16_kernel<64, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((attn_bf16_kernel<64, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

// ----------------------------------------------------------------- fp32 path
// Four lanes per query row, each holding D/4 dims of q and of the output;
// keys are streamed from global memory (broadcast within the workgroup).
constexpr int kF32Queries = 64;

template <int D, bool PART>
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
  constexpr int DL = D / 4;
  const int part = PART ? blockIdx.z : 0;
  const int bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
  const int N = a.N;
  const int tid = threadIdx.x, sub = tid & 3;
  const int qrow = blockIdx.x * kF32Queries + (tid >> 2);
  const bool qvalid = qrow < N;
  const int qr = qvalid ? qrow : N - 1;
  const float* qp = static_cast<const float*>(a.q) + b * a.q_sb + h * a.q_sh + (int64_t)qr * a.q_sn + sub * DL;
  const float* kg = static_cast<const float*>(a.k) + b * a.k_sb + h * a.k_sh + sub * DL;
  const float* vg = static_cast<const float*>(a.v) + b * a.v_sb + h * a.v_sh + sub * DL;
  float qv[DL], ov[DL];
#pragma unroll
  for (int i = 0; i < DL; i += 4) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(qp + i);
    qv[i] = x[0]; qv[i + 1] = x[1]; qv[i + 2] = x[2]; qv[i + 3] = x[3];
    ov[i] = ov[i + 1] = ov[i + 2] = ov[i + 3] = 0.0f;
  }
  const float tq = a.tq[(int64_t)b * N + qr];
  const float mq = a.mq[(int64_t)b * N + qr];
  const float* tkb = a.tk + (int64_t)b * a.npad;
  const float* kbb = a.kb + (int64_t)b * a.npad;
  const int k0 = a.kr[part], k1 = a.kr[part + 1];
  float m = -INFINITY, l = 0.0f;
  for (int kx = k0; kx < k1; ++kx) {
    const float* kp = kg + (int64_t)kx * a.k_sn;
    float sdot = 0.0f;
#pragma unroll
    for (int i = 0; i < DL; i += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(kp + i);
      sdot = fmaf(qv[i], x[0], sdot);
      sdot = fmaf(qv[i + 1], x[1], sdot);
      sdot = fmaf(qv[i + 2], x[2], sdot);
      sdot = fmaf(qv[i + 3], x[3], sdot);
    }
    sdot += __shfl_xor(sdot, 1);
    sdot += __shfl_xor(sdot, 2);
    const float dd = fmaxf(fmaf(fabsf(tq - tkb[kx]), a.sigma, -a.w), 0.0f);
    const float x = fmaf(sdot, a.c, fmaf(mq, kbb[kx], -fminf(dd * dd, a.cap2)));
    const float mn = fmaxf(m, x);
    const float alpha = exp2f(m - mn);
    const float p = exp2f(x - mn);
    l = fmaf(l, alpha, p);
    const float* vp = vg + (int64_t)kx * a.v_sn;
#pragma unroll
    for (int i = 0; i < DL; i += 4) {
      const f32x4 vv = *reinterpret_cast<const f32x4*>(vp + i);
      ov[i] = fmaf(ov[i], alpha, p * vv[0]);
      ov[i + 1] = fmaf(ov[i + 1], alpha, p * vv[1]);
      ov[i + 2] = fmaf(ov[i + 2], alpha, p * vv[2]);
      ov[i + 3] = fmaf(ov[i + 3], alpha, p * vv[3]);
    }
    m = mn;
  }
  if (!qvalid) return;
  const bool empty = k1 <= k0;
  const float inv = empty ? 0.0f : 1.0f / l;
  const float lse = empty ? -INFINITY : (m + log2f(l)) * kLn2;
  float* op;
  if (PART) op = a.opart + ((((int64_t)part * a.B + b) * a.H + h) * N + qrow) * D + sub * DL;
  else op = static_cast<float*>(a.o) + b * a.o_sb + h * a.o_sh + (int64_t)qrow * a.o_sn + sub * DL;
#pragma unroll
  for (int i = 0; i < DL; i += 4)
    *reinterpret_cast<f32x4*>(op + i) = f32x4{ov[i] * inv, ov[i + 1] * inv, ov[i + 2] * inv, ov[i + 3] * inv};
  if (sub == 0) {
    if (PART) a.lsepart[(((int64_t)part * a.B + b) * a.H + h) * N + qrow] = lse;
    else a.lse[((int64_t)b * a.H + h) * N + qrow] = lse;
  }
}

int attn_f32_block_q(int) { return kF32Queries; }

hipError_t launch_attn_f32(const AttnArgs& a, int D, bool partitioned, hipStream_t s) {
  dim3 grid((a.N + kF32Queries - 1) / kF32Queries, a.B * a.H, partitioned ? a.nparts : 1);
  dim3 block(256);
  if (D == 128) {
    if (partitioned) hipLaunchKernelGGL((attn_f32_kernel<128, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((attn_f32_kernel<128, false>), grid, block, 0, s, a);
  } else {
    if (partitioned) hipLaunchKernelGGL((attn_f32_kernel<64, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((attn_f32_kernel<64, false>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

// --------------------------------------------------------------- LSE merge
// One thread per (row, 4 consecutive dims).
template <bool BF16_OUT>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int dq = a.D / 4;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rows = (int64_t)a.B * a.H * a.N;
  if (gid >= rows * dq) return;
  const int d4 = (int)(gid % dq);
  const int64_t row = gid / dq;                   // (b*H + h)*N + n
  const int n = (int)(row % a.N);
  const int64_t bh = row / a.N;
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  float mx = -INFINITY;
  for (int p = 0; p < a.nparts; ++p) mx = fmaxf(mx, a.lsepart[(int64_t)p * rows + row]);
  float ssum = 0.0f;
  for (int p = 0; p < a.nparts; ++p) ssum += expf(a.lsepart[(int64_t)p * rows + row] - mx);
  const float lse = mx + logf(ssum);
  f32x4 acc = f32x4{};
  for (int p = 0; p < a.nparts; ++p) {
    const float w = expf(a.lsepart[(int64_t)p * rows + row] - lse);
    const f32x4 x = *reinterpret_cast<const f32x4*>(a.opart + ((int64_t)p * rows + row) * a.D + d4 * 4);
    acc += w * x;
  }
  const int64_t oo = b * a.o_sb + h * a.o_sh + (int64_t)n * a.o_sn + d4 * 4;
  if (BF16_OUT) {
    bf16x4 y;
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = (__bf16)acc[i];
    *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(a.o) + oo) = y;
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + oo) = acc;
  }
  if (d4 == 0) a.lse[row] = lse;
}

hipError_t launch_merge(const MergeArgs& a, bool bf16_out, hipStream_t s) {
  const int64_t total = (int64_t)a.B * a.H * a.N * (a.D / 4);
  dim3 grid((unsigned)((total + 255) / 256));
  if (bf16_out) hipLaunchKernelGGL(merge_kernel<true>, grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL(merge_kernel<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace tara
