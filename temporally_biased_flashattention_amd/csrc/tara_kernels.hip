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
// Lazy rescaling threshold (log2 units): the reference m used in the exponent
// only moves when a row's logits may exceed it by more than this, so the
// unnormalised probabilities stay <= 2^20 (far from fp32 / bf16 overflow;
// relative precision does not depend on the scale).
constexpr float kRescaleTau = 20.0f;

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

// ------------------------------------------------------ key-tile norm bound
// kmax[b*H + h][t] = max |k_n| over the 64 keys of tile t (rows past N repeat
// row N-1, as the attention kernel's staging does). 256 threads per tile: four
// adjacent threads read one row's D/4 contiguous elements (coalesced), the
// row's sum of squares is combined across them, then the max over the rows.
__global__ __launch_bounds__(256) void knorm_kernel(const __bf16* __restrict__ k, int64_t sb, int64_t sh, int64_t sn,
                                                    int H, int N, int D, int nkt, float* __restrict__ kmax) {
  __shared__ float wmax[4];
  const int t = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H;
  const int r = threadIdx.x >> 2, qd = threadIdx.x & 3;
  const int n = min(t * kBlockK + r, N - 1);
  const int dq = D / 4;
  const __bf16* kp = k + b * sb + h * sh + (int64_t)n * sn + qd * dq;
  float ss = 0.0f;
  for (int i = 0; i < dq; i += 8) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(kp + i);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float f = (float)v[e];
      ss = fmaf(f, f, ss);
    }
  }
  ss += __shfl_xor(ss, 1);
  ss += __shfl_xor(ss, 2);
  float m = sqrtf(ss);
  for (int off = 32; off >= 4; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    kmax[(int64_t)bh * nkt + t] = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
}

hipError_t launch_knorm(const __bf16* k, int64_t sb, int64_t sh, int64_t sn, float* kmax, int B, int H, int N,
                        int nkt, int D, hipStream_t s) {
  dim3 grid(nkt, B * H);
  hipLaunchKernelGGL(knorm_kernel, grid, dim3(256), 0, s, k, sb, sh, sn, H, N, D, nkt, kmax);
  return hipGetLastError();
}

// --------------------------------------------------------- bf16 MFMA kernel
// One workgroup = NW waves x 32 query rows of one (batch, head). Per 64-key
// tile t every wave runs a two-phase software pipeline so that its MFMAs and
// its softmax VALU work interleave in program order (MFMA and VALU of one wave
// co-issue; in-order issue means the VALU work has to sit between the MFMAs):
//   phase A: S_{t+1} = K_{t+1} Q^T (16 MFMAs)   with   P_t = exp2(X_t), row sums, bf16 pack
//   phase B: O^T += V_t^T P_t^T (16 MFMAs)      with   max / bias class / X_{t+1} = S_{t+1} c + b - m
// so K runs one tile ahead of V in LDS: iteration t reads K_{t+1} and V_t and
// stages K_{t+2} and V_{t+1} (two LDS buffers each, one barrier per tile).

// LDS ring depth of the bf16 kernel (K/V^T tile pairs in flight).
constexpr int kStages = 3;

// Key row held by S^T output row `r` of a 32-key block: bits 2 and 3 swapped.
__device__ __forceinline__ int perm32(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// A byte range of global memory addressed by buffer instructions (raw
// addressing, stride 0): loads past `bytes` return zeros instead of touching
// other memory.
struct BufRange {
  const void* base;
  uint32_t bytes;
};

// 16 bytes per lane from r.base + soff + voff into LDS at lds + 16 * lane.
__device__ __forceinline__ void dma16(BufRange r, uint32_t voff, uint32_t soff, char* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(r.base), 0, (int)r.bytes, 0x00020000),
      (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

// Tile staging by LDS DMA (buffer_load_dwordx4 ... lds): one wave instruction
// writes 64 lanes x 16 bytes contiguously at a uniform LDS address. Every call
// stages one padded K tile (64 rows of KROWB bytes) and one padded V^T tile
// (D rows of VROWB bytes) as whole 1-KB blocks: combined block ci < KBLK is K,
// the rest V^T, and wave w takes blocks w, w + NW, ... (PER_MAX DMAs for waves
// w < TOT % NW, PER_MIN for the others). A lane whose 16 bytes fall on a row's
// pad chunk re-reads chunk 0 of its row (never read back). Buffer loads rather
// than global_load_lds: the latter is FLAT-encoded, and while one is in flight
// the compiler cannot count LDS reads, so every fragment wait drains them all.
template <int KROWB, int KDATA, int KBLK, int VROWB, int VDATA, int VBLK, int NW>
struct KvDma {
  static constexpr int TOT = KBLK + VBLK;
  static constexpr int PER_MIN = TOT / NW;
  static constexpr int PER_MAX = (TOT + NW - 1) / NW;
  static constexpr int NEXTRA = TOT % NW;   // waves issuing PER_MAX
  uint32_t voff[PER_MAX];   // byte offset of this lane's 16 bytes in its tile
  int krow[PER_MAX];        // K tile row of those bytes (tail clamp)
  __device__ void init(int wave, int lane, uint32_t k_row_bytes, uint32_t v_row_bytes) {
#pragma unroll
    for (int p = 0; p < PER_MAX; ++p) {
      const int ci = min(wave + p * NW, TOT - 1);
      if (ci < KBLK) {
        const int o = ci * 1024 + lane * 16, r = o / KROWB, c = (o % KROWB) / 16;
        krow[p] = r;
        voff[p] = r * k_row_bytes + (c < KDATA ? c * 16 : 0);
      } else {
        const int o = (ci - KBLK) * 1024 + lane * 16, d = o / VROWB, c = (o % VROWB) / 16;
        krow[p] = 0;
        voff[p] = d * v_row_bytes + (c < VDATA ? c * 16 : 0);
      }
    }
  }
  // DMAs this wave issues per call (uniform)
  __device__ static int count(int wave) { return wave < NEXTRA ? PER_MAX : PER_MIN; }
  // K rows past the sequence (tail tile, rows_left < 64) re-read its last
  // row; those keys are masked later. wave must be in [0, NW).
  __device__ void issue(BufRange rk, uint32_t ksoff, int rows_left, uint32_t k_row_bytes, char* lds_k, BufRange rv,
                        uint32_t vsoff, char* lds_v, int wave) const {
    if (rows_left >= kBlockK) issue_blocks<false>(rk, ksoff, rows_left, k_row_bytes, lds_k, rv, vsoff, lds_v, wave);
    else issue_blocks<true>(rk, ksoff, rows_left, k_row_bytes, lds_k, rv, vsoff, lds_v, wave);
  }
  template <bool TAIL>
  __device__ void issue_blocks(BufRange rk, uint32_t ksoff, int rows_left, uint32_t k_row_bytes, char* lds_k,
                               BufRange rv, uint32_t vsoff, char* lds_v, int wave) const {
#pragma unroll
    for (int p = 0; p < PER_MAX; ++p) {
      if (p >= PER_MIN && wave >= NEXTRA) break;
      const int ci = wave + p * NW;
      // decided at compile time unless the blocks of step p straddle K and V^T
      const bool isk = (p + 1) * NW <= KBLK ? true : p * NW >= KBLK ? false : ci < KBLK;
      if (isk) {
        uint32_t vo = voff[p];
        if (TAIL) vo -= (uint32_t)(krow[p] - min(krow[p], rows_left - 1)) * k_row_bytes;
        dma16(rk, vo, ksoff, lds_k + ci * 1024);
      } else {
        dma16(rv, voff[p], vsoff, lds_v + (ci - KBLK) * 1024);
      }
    }
  }
};

// Wait until at most KEEP of this wave's vector-memory operations are pending
// (the newest KEEP DMAs may stay in flight).
template <int KEEP>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(KEEP) : "memory");
}

// S^T for the two 32-key blocks of a K tile in LDS.
template <int D, int KROW>
__device__ __forceinline__ void qk_tile(f32x16 (&s)[2], const __bf16* ks, int krow_lane, int hh,
                                        const bf16x8 (&qf)[D / 16]) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    s[kb] = f32x16{};
    const __bf16* kr = ks + (kb * 32 + krow_lane) * KROW + hh * 8;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(kr + kk * 16), qf[kk],
                                                      s[kb], 0, 0, 0);
  }
}

// i-th K fragment of phase A: key block i & 1, head-dim step i >> 1.
template <int KROW>
__device__ __forceinline__ bf16x8 kfrag(const __bf16* kr0, int i) {
  return *reinterpret_cast<const bf16x8*>(kr0 + (i & 1) * 32 * KROW + (i >> 1) * 16);
}

// i-th V^T fragment of phase B: 32-row block i % NDB of the head dim, 16-key
// chunk i / NDB (key block kb = chunk / 2, half c2 = chunk % 2).
template <int VROW, int NDB>
__device__ __forceinline__ bf16x8 vfrag(const __bf16* vr0, int i) {
  return *reinterpret_cast<const bf16x8*>(vr0 + (i % NDB) * 32 * VROW + (i / NDB) * 16);
}

// max of three floats as one v_max3_f32. The operands here are scores (finite,
// or -inf for masked keys), so the NaN quieting that fmaxf adds around MFMA
// results (one extra v_max_f32 per operand) is not needed.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(unsigned, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 w) { return __builtin_bit_cast(bf16x8, w); }

// Marks 16 values as used at this point (emits no instruction). The operands
// are single floats: a 64-byte vector operand is not valid for the host pass,
// which then silently drops the kernel's launch stub.
__device__ __forceinline__ void keep16(const f32x16& v) {
  asm volatile("" ::"v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]), "v"(v[4]), "v"(v[5]), "v"(v[6]), "v"(v[7]),
               "v"(v[8]), "v"(v[9]), "v"(v[10]), "v"(v[11]), "v"(v[12]), "v"(v[13]), "v"(v[14]), "v"(v[15]));
}

typedef const __attribute__((address_space(4))) KeyTileSummary* KsumConstPtr;

// Uniform load of a tile summary through the constant address space (scalar loads).
__device__ __forceinline__ KeyTileSummary load_summary(KsumConstPtr p, int i) {
  KeyTileSummary r;
  r.kind = p[i].kind;
  r.lo = p[i].lo;
  r.hi = p[i].hi;
  r.bias = p[i].bias;
  return r;
}

// Bias class of one key tile for one query row: returns true when the tile
// needs the per-element formula for this row; otherwise *brow is the row's
// constant bias over the tile (log2 units).
__device__ __forceinline__ bool tile_class_lane(const KeyTileSummary& sm, bool partial, bool qbiased, float tq,
                                                float mq, const AttnArgs& a, float* brow) {
  float b = 0.0f;
  bool lane_elem = partial;
  if (!partial) {
    if (sm.kind == KT_GUIDE) {
      if (qbiased) {
        const float dlo = sm.lo - tq, dhi = tq - sm.hi;
        const float dmin = fmaxf(fmaxf(dlo, dhi), 0.0f);
        const float dmax = fmaxf(-dlo, -dhi);
        if (dmin >= a.dsat) b = -a.cap2;
        else if (!(dmax <= a.window)) lane_elem = true;
      }
    } else if (sm.kind == KT_PICTURE) {
      b = mq * sm.bias;
    } else if (sm.kind == KT_MIXED) {
      lane_elem = true;
    }
  }
  *brow = b;
  return lane_elem;
}

// Per-element bias of a key tile, in place: x = s*c + m*log2(gain) - penalty,
// keys outside [k0, k1) -> -inf. Lane half hh holds keys 8*hh..8*hh+7 and
// 16+8*hh..16+8*hh+7 of each 32-key block.
__device__ __forceinline__ void elem_bias(f32x16 (&s)[2], int kbase, int hh, float tq, float mq, bool partial, int k0,
                                          int k1, const float* tkb, const float* kbb, const AttnArgs& a) {
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
}

template <int D, int NW, int QB, bool PART>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4)))
void attn_bf16_kernel(AttnArgs a) {
  constexpr int BQ = NW * QB * 32;         // query rows per workgroup
  constexpr int KROW = D + 8;              // padded LDS pitch of a K row (elements)
  constexpr int VROW = kBlockK + 8;        // padded LDS pitch of a V^T row (elements)
  constexpr int KTILE = kBlockK * KROW;
  constexpr int VTILE = D * VROW;
  constexpr int NKK = D / 16;
  constexpr int NDB = D / 32;
  // LDS ring of NS stages: K tiles in slots 0..NS-1, then V^T tiles in slots 0..NS-1
  constexpr int NS = kStages;
  __shared__ __attribute__((aligned(16))) __bf16 smem[NS * (KTILE + VTILE)];
#define KBUF(i) (smem + (i) * KTILE)
#define VBUF(i) (smem + NS * KTILE + (i) * VTILE)

  const int part = PART ? blockIdx.y : 0;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = L / a.nqb, qblk = L % a.nqb;
  const int b = bh / a.H, h = bh % a.H;
  const int N = a.N;

  const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (NW - 1);   // uniform per wave

  // this lane's query rows: block q of the wave holds rows wave*32*QB + 32*q + lq
  int qrow[QB];
  bool qvalid[QB];
  bf16x8 qf[QB][NKK];
  float tq[QB], mq[QB];
  bool qbiased[QB];
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    qrow[q] = qblk * BQ + (wave * QB + q) * 32 + lq;
    qvalid[q] = qrow[q] < N;
    const int qr = qvalid[q] ? qrow[q] : N - 1;
    const __bf16* qp = static_cast<const __bf16*>(a.q) + b * a.q_sb + h * a.q_sh + (int64_t)qr * a.q_sn;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qf[q][kk] = *reinterpret_cast<const bf16x8*>(qp + kk * 16 + hh * 8);
    tq[q] = a.tq[(int64_t)b * N + qr];
    mq[q] = a.mq[(int64_t)b * N + qr];
    qbiased[q] = tq[q] == tq[q];
  }

  const int k0 = a.kr[part], k1 = a.kr[part + 1];
  if (k1 <= k0) {
    // empty key range (partitioned mode only): contributes nothing to the merge
    if (PART) {
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        if (!qvalid[q]) continue;
        float* op = a.opart + ((((int64_t)part * a.B + b) * a.H + h) * N + qrow[q]) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) *reinterpret_cast<f32x4*>(op + db * 32 + j * 8 + hh * 4) = f32x4{};
        if (hh == 0) a.lsepart[(((int64_t)part * a.B + b) * a.H + h) * N + qrow[q]] = -INFINITY;
      }
    }
    return;
  }
  const int kt0 = k0 / kBlockK, kt1 = (k1 + kBlockK - 1) / kBlockK;

  // staging: buffer resources over this head's K rows and V^T rows; per-lane
  // 32-bit offsets within a tile, per-tile scalar offsets
  const __bf16* kg = static_cast<const __bf16*>(a.k) + b * a.k_sb + h * a.k_sh;
  const __bf16* vg = a.vt + (int64_t)bh * D * a.npad;
  const uint32_t k_sn_bytes = (uint32_t)(a.k_sn * 2);
  const BufRange rk{kg, (uint32_t)(N - 1) * k_sn_bytes + D * 2};
  const BufRange rv{vg, (uint32_t)(D * a.npad * 2)};
  constexpr int KBLK = KTILE * 2 / 1024, VBLK = VTILE * 2 / 1024;
  static_assert(KBLK * 1024 == KTILE * 2 && VBLK * 1024 == VTILE * 2, "tiles are whole 1-KB blocks");
  using Dma = KvDma<KROW * 2, D / 8, KBLK, VROW * 2, kBlockK / 8, VBLK, NW>;
  Dma dma;
  dma.init(wave, lane, k_sn_bytes, (uint32_t)a.npad * 2);
  const bool dma_extra = Dma::count(wave) == Dma::PER_MAX;
  // stage K tile kk into K slot sk and V^T tile kv into V slot sv (indices past
  // the range are clamped to its last tile: the slot is free either way)
  auto stage = [&](int kk, int sk, int kv, int sv) {
    kk = min(kk, kt1 - 1);
    kv = min(kv, kt1 - 1);
    dma.issue(rk, (uint32_t)kk * kBlockK * k_sn_bytes, N - kk * kBlockK, k_sn_bytes,
              reinterpret_cast<char*>(KBUF(sk)), rv, (uint32_t)kv * kBlockK * 2, reinterpret_cast<char*>(VBUF(sv)),
              wave);
  };
  // keep this iteration's DMAs (and those of the NS-3 before it) in flight
  auto wait_staged = [&]() {
    if (dma_extra) wait_vm<(NS - 2) * Dma::PER_MAX>();
    else wait_vm<(NS - 2) * Dma::PER_MIN>();
  };

  const float* tkb = a.tk + (int64_t)b * a.npad;
  const float* kbb = a.kb + (int64_t)b * a.npad;
  const KeyTileSummary* ks_b = a.ksum + (int64_t)b * a.nkt;
  // the same summaries through the constant address space: uniform loads of
  // them become scalar loads
  const KsumConstPtr ks_c = (KsumConstPtr)ks_b;
  const int krow_lane = perm32(lq);
  KeyTileSummary sm_next;
  // max over each key tile of |k| (this head), for the row-max bound
  const __attribute__((address_space(4))) float* kmax_c =
      (const __attribute__((address_space(4))) float*)(a.kmax + (int64_t)bh * a.nkt);
  float kmax_next;
  // |q| * c, rounded up by 2^-10 to cover fp32 rounding of the MFMA sum
  float qn_c[QB];
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    float ss = 0.0f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = (float)qf[q][kk][e];
        ss = fmaf(v, v, ss);
      }
    qn_c[q] = sqrtf(xor32_sum(ss)) * a.c * (1.0f + 0x1.0p-10f);
  }

  f32x16 o[QB][NDB];
#pragma unroll
  for (int q = 0; q < QB; ++q)
#pragma unroll
    for (int i = 0; i < NDB; ++i) o[q][i] = f32x16{};
  float m_used[QB], lsum[QB];
  f32x16 x[QB][2];   // X_t = S_t * c + bias - m_used (exp2 argument)
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    m_used[q] = -INFINITY;
    lsum[q] = 0.0f;
  }

  {
    // prologue: K and V^T of tiles t0 .. t0+NS-1 into slots 0 .. NS-1; S_t0; X_t0
#pragma unroll
    for (int i = 0; i < NS; ++i) stage(kt0 + i, i, kt0 + i, i);
    wait_vm<0>();
    __builtin_amdgcn_s_barrier();
#pragma unroll
    for (int q = 0; q < QB; ++q) qk_tile<D, KROW>(x[q], KBUF(0), krow_lane, hh, qf[q]);
    const int kbase = kt0 * kBlockK;
    const bool partial = kbase < k0 || kbase + kBlockK > k1;
    const KeyTileSummary sm0 = load_summary(ks_c, kt0);
    float brow[QB];
    bool lane_elem = false;
#pragma unroll
    for (int q = 0; q < QB; ++q) lane_elem |= tile_class_lane(sm0, partial, qbiased[q], tq[q], mq[q], a, &brow[q]);
    float cc = a.c;
    if (wave_any(lane_elem)) {
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        elem_bias(x[q], kbase, hh, tq[q], mq[q], partial, k0, k1, tkb, kbb, a);
        brow[q] = 0.0f;
      }
      cc = 1.0f;
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      float mx = x[q][0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, x[q][kb][r]);
      m_used[q] = fmaf(xor32_max(mx), cc, brow[q]);
      const float off = brow[q] - m_used[q];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) x[q][kb][r] = fmaf(x[q][kb][r], cc, off);
    }
    sm_next = load_summary(ks_c, min(kt0 + 1, kt1 - 1));
    kmax_next = kmax_c[min(kt0 + 1, kt1 - 1)];
    // every wave is done with K slot 0 before iteration 0 restages it
    __builtin_amdgcn_s_barrier();
  }

  // ring slots: iteration t reads K_{t+1} (slot s1) and V_t (slot s0), and
  // restages K_{t+NS} into slot s0 (K_t's, read last iteration) and
  // V_{t+NS-1} into slot sprev (V_{t-1}'s, read last iteration)
  int s0 = 0;
  for (int t = kt0; t < kt1; ++t) {
    const bool has1 = t + 1 < kt1;
    const int s1 = s0 + 1 == NS ? 0 : s0 + 1;
    const int sprev = s0 == 0 ? NS - 1 : s0 - 1;
    stage(t + NS, s0, t + NS - 1, sprev);
    const __bf16* kn = KBUF(s1);
    const __bf16* vc = VBUF(s0);
    const int kbase1 = (t + 1) * kBlockK;
    const bool partial1 = kbase1 < k0 || kbase1 + kBlockK > k1;
    const KeyTileSummary sm1 = sm_next;
    const float kmax1 = kmax_next;

    // phase A: S_{t+1} = K_{t+1} Q^T (each K fragment feeds the QB query
    // blocks; the two 32-key blocks alternate) | P_t = exp2(X_t) in place and
    // its bf16 pack. K fragments are read from LDS three fragments ahead.
    f32x16 sn[QB][2];
#pragma unroll
    for (int q = 0; q < QB; ++q) sn[q][0] = sn[q][1] = f32x16{};
    const __bf16* kr0 = kn + krow_lane * KROW + hh * 8;
    bf16x8 kf[4];
    kf[0] = kfrag<KROW>(kr0, 0);
    kf[1] = kfrag<KROW>(kr0, 1);
    kf[2] = kfrag<KROW>(kr0, 2);
    u32x4 pw[QB][4];   // P_t as packed bf16 pairs: pw[q][kb*2 + c2] is the B operand of PV block (kb, c2)
    auto exp_pair = [&](int q, int i) {
      // elements 2i, 2i+1 of the lane's 32 scores of tile t (query block q)
      const int kb = i >> 3, r = (2 * i) & 15;
      const float p0 = fast_exp2(x[q][kb][r]), p1 = fast_exp2(x[q][kb][r + 1]);
      x[q][kb][r] = p0;
      x[q][kb][r + 1] = p1;
      pw[q][i >> 2][i & 3] = pack_bf16x2(p0, p1);
    };
#pragma unroll
    for (int i = 0; i < 2 * NKK; ++i) {
      if (i + 3 < 2 * NKK) kf[(i + 3) & 3] = kfrag<KROW>(kr0, i + 3);
#pragma unroll
      for (int q = 0; q < QB; ++q)
        sn[q][i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i & 3], qf[q][i >> 1], sn[q][i & 1], 0, 0, 0);
      if (i < 16) {
#pragma unroll
        for (int q = 0; q < QB; ++q) exp_pair(q, i);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 2 * NKK; i < 16; ++i)
#pragma unroll
      for (int q = 0; q < QB; ++q) exp_pair(q, i);
    // keep P_t in this block (the PV product that reads it follows the
    // bias-class branch)
#pragma unroll
    for (int q = 0; q < QB; ++q) asm volatile("" ::"v"(pw[q][0]), "v"(pw[q][1]), "v"(pw[q][2]), "v"(pw[q][3]));

    // bias class of tile t+1 (rare per-element path before phase B)
    float brow[QB];
    float cc = a.c;
    bool need_max = false;
#pragma unroll
    for (int q = 0; q < QB; ++q) brow[q] = 0.0f;
    if (has1) {
      bool lane_elem = false;
#pragma unroll
      for (int q = 0; q < QB; ++q)
        lane_elem |= tile_class_lane(sm1, partial1, qbiased[q], tq[q], mq[q], a, &brow[q]);
      if (wave_any(lane_elem)) {
#pragma unroll
        for (int q = 0; q < QB; ++q) {
          elem_bias(sn[q], kbase1, hh, tq[q], mq[q], partial1, k0, k1, tkb, kbb, a);
          brow[q] = 0.0f;
        }
        cc = 1.0f;
        need_max = true;
      } else {
        // every logit of the tile is <= |q| max|k| c + brow (Cauchy-Schwarz);
        // the exact row max is needed only when that bound could pass m + tau
        bool lane_need = false;
#pragma unroll
        for (int q = 0; q < QB; ++q) lane_need |= fmaf(qn_c[q], kmax1, brow[q]) > m_used[q] + kRescaleTau;
        need_max = wave_any(lane_need);
      }
    }
    float m_new[QB], off[QB];
#pragma unroll
    for (int q = 0; q < QB; ++q) m_new[q] = m_used[q];
    if (need_max) {
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        float mxa = -INFINITY, mxb = -INFINITY;
#pragma unroll
        for (int f = 0; f < 32; f += 4) {
          mxa = max3f(mxa, sn[q][f >> 4][f & 15], sn[q][f >> 4][(f & 15) + 1]);
          mxb = max3f(mxb, sn[q][f >> 4][(f & 15) + 2], sn[q][f >> 4][(f & 15) + 3]);
        }
        const float mt = fmaf(xor32_max(fmaxf(mxa, mxb)), cc, brow[q]);
        if (mt > m_used[q] + kRescaleTau) m_new[q] = mt;
      }
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) off[q] = brow[q] - m_new[q];

    // phase B: O^T += V_t^T P_t^T (each V^T fragment feeds the QB query
    // blocks) | row sum of P_t, X_{t+1} = S_{t+1} c + brow - m_new. V^T
    // fragments are read three fragments ahead.
    const __bf16* vr0 = vc + lq * VROW + hh * 8;
    bf16x8 vf[4];
    vf[0] = vfrag<VROW, NDB>(vr0, 0);
    vf[1] = vfrag<VROW, NDB>(vr0, 1);
    vf[2] = vfrag<VROW, NDB>(vr0, 2);
    float ts[QB][2];
#pragma unroll
    for (int q = 0; q < QB; ++q) ts[q][0] = ts[q][1] = 0.0f;
#pragma unroll
    for (int i = 0; i < 4 * NDB; ++i) {
      if (i + 3 < 4 * NDB) vf[(i + 3) & 3] = vfrag<VROW, NDB>(vr0, i + 3);
      const int db = i % NDB, kc = i / NDB;
#pragma unroll
      for (int q = 0; q < QB; ++q)
        o[q][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i & 3], as_bf16x8(pw[q][kc]), o[q][db], 0, 0, 0);
      // spread 32 sums and 32 scale-FMAs per query block over the fragments
      constexpr int NM = 4 * NDB;
      constexpr int PER = (32 + NM - 1) / NM;
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int f = i * PER + u;
        if (f < 32) {
#pragma unroll
          for (int q = 0; q < QB; ++q) {
            ts[q][f & 1] += x[q][f >> 4][f & 15];
            x[q][f >> 4][f & 15] = fmaf(sn[q][f >> 4][f & 15], cc, off[q]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // X_{t+1} belongs to phase B (its FMAs hide under the PV MFMAs): keep it
    // from being sunk past the rescale branch
#pragma unroll
    for (int q = 0; q < QB; ++q)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) keep16(x[q][kb]);
    bool any_grow = false;
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      lsum[q] += ts[q][0] + ts[q][1];
      any_grow |= m_new[q] > m_used[q];
    }
    if (wave_any(any_grow)) {
      // lazy rescale after the PV product of tile t (which used the old m)
#pragma unroll
      for (int q = 0; q < QB; ++q) {
        const float alpha = fast_exp2(m_used[q] - m_new[q]);
        lsum[q] *= alpha;
#pragma unroll
        for (int i = 0; i < NDB; ++i) o[q][i] *= alpha;
        m_used[q] = m_new[q];
      }
    }

    // K_{t+2} and V_{t+1} (staged NS-2 iterations ago) have landed; newer DMAs may fly on
    wait_staged();
    sm_next = load_summary(ks_c, min(t + 2, kt1 - 1));
    kmax_next = kmax_c[min(t + 2, kt1 - 1)];
    __builtin_amdgcn_s_barrier();
    // take the scalar loads here, where no LDS read is pending: a scalar load
    // still in flight would turn every LDS fragment wait of the next
    // iteration into a full drain (scalar loads complete out of order)
    asm volatile("" ::"s"(sm_next.kind), "s"(sm_next.lo), "s"(sm_next.hi), "s"(sm_next.bias), "s"(kmax_next));
    s0 = s1;
  }
  // no DMA may still target this workgroup's LDS when it exits
  wait_vm<0>();

  // epilogue
#pragma unroll
  for (int q = 0; q < QB; ++q) {
    const float ltot = xor32_sum(lsum[q]);
    if (!qvalid[q]) continue;
    const float inv = 1.0f / ltot;
    const float lse = (m_used[q] + __log2f(ltot)) * kLn2;
    if (PART) {
      float* op = a.opart + ((((int64_t)part * a.B + b) * a.H + h) * N + qrow[q]) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f32x4 y;
#pragma unroll
          for (int i = 0; i < 4; ++i) y[i] = o[q][db][j * 4 + i] * inv;
          *reinterpret_cast<f32x4*>(op + db * 32 + j * 8 + hh * 4) = y;
        }
      if (hh == 0) a.lsepart[(((int64_t)part * a.B + b) * a.H + h) * N + qrow[q]] = lse;
    } else {
      __bf16* op = static_cast<__bf16*>(a.o) + b * a.o_sb + h * a.o_sh + (int64_t)qrow[q] * a.o_sn;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          bf16x4 y;
#pragma unroll
          for (int i = 0; i < 4; ++i) y[i] = (__bf16)(o[q][db][j * 4 + i] * inv);
          *reinterpret_cast<bf16x4*>(op + db * 32 + j * 8 + hh * 4) = y;
        }
      if (hh == 0) a.lse[((int64_t)b * a.H + h) * N + qrow[q]] = lse;
    }
  }
}

#undef KBUF
#undef VBUF

// Workgroup shape of the bf16 kernel: kWaves waves, each owning kQB blocks of
// 32 query rows (every LDS fragment then feeds kQB MFMAs).
constexpr int kWaves = 8;
constexpr int kQB = 1;

int attn_bf16_block_q(int) { return kWaves * kQB * 32; }

int attn_bf16_grid(const AttnArgs& a) { return a.nqb * a.B * a.H; }

hipError_t launch_attn_bf16(const AttnArgs& a, int D, bool partitioned, hipStream_t s) {
  dim3 grid(attn_bf16_grid(a), partitioned ? a.nparts : 1);
  dim3 block(kWaves * 64);
  if (D == 128) {
    if (partitioned) hipLaunchKernelGGL((attn_bf16_kernel<128, kWaves, kQB, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((attn_bf16_kernel<128, kWaves, kQB, false>), grid, block, 0, s, a);
  } else {
    if (partitioned) hipLaunchKernelGGL((attn_bf16_kernel<64, kWaves, kQB, true>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((attn_bf16_kernel<64, kWaves, kQB, false>), grid, block, 0, s, a);
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
