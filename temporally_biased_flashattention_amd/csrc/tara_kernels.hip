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
//   knorm_kernel       max |k| per 64-key tile (the row-max bound of the bf16 pass)
//   kquant_kernel      8-bit Q.K: K in FP8 E4M3 with one power-of-two scale per
//                      tile, plus the tile norms
//   dense_bias_kernel  the dense-bias baseline: every logit's bias written out
//   attn_bf16_kernel   the fused pass: bf16 MFMA S^T = K Q^T, bias, online
//                      softmax, MFMA O^T += V^T P^T, one workgroup per block
//                      of query rows of one (batch, head), streaming all key
//                      tiles of its key range through LDS; its variants serve
//                      key-range partitions, the three term passes, 8-bit Q.K
//                      and the dense-bias baseline
//   attn_f32_kernel    fp32 inputs: same arithmetic with FMA, K/V tiles staged in LDS
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
#include <float.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

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

// Sum over the four lanes of a quad (lanes 4r .. 4r+3), by DPP quad permutes
// (lane ^ 1, then lane ^ 2); every lane of the quad must be active.
__device__ __forceinline__ float quad_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
  return x;
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
  const int64_t plane = a.mask_plane;   // mask plane stride
  int seg = valid ? (int)a.seg[mi] : 3;
  const float t = valid ? a.time[mi] : 0.0f;
  const bool tfinite = valid && isfinite(t);
  const float nanv = __builtin_nanf("");

  // query side (n < N only)
  if (valid) {
    const bool tgt = seg == 0;
    a.tq[mi] = (tgt && a.bias_active && tfinite) ? t : nanv;
    const bool bq = tgt && a.binding_active;
    // summed log2 gains of this query for every picture: sum_j m_j * log2 gain_j,p
    if (a.num_pictures > 0) {
      // a non-finite mask weight drops that binding's term for this query
      float m[kMaxBindings];
#pragma unroll
      for (int j = 0; j < kMaxBindings; ++j) {
        m[j] = (bq && j < a.nbind) ? (a.mask ? a.mask[j * plane + mi] : 1.0f) : 0.0f;
        if (!isfinite(m[j])) m[j] = 0.0f;
      }
      float* g = a.gt + mi * a.num_pictures;
      for (int p = 0; p < a.num_pictures; ++p) {
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < kMaxBindings; ++j)
          if (j < a.nbind) acc = fmaf(m[j], a.lg2gain[j][p], acc);
        g[p] = acc;
      }
    }
  }
  // key side (n < npad)
  const bool isg = valid && seg == 1 && a.bias_active && tfinite;
  const float tk = isg ? t : nanv;
  int kp = -1;
  if (valid && seg == 2 && a.binding_active) {
    const int id = a.pic[mi];
    if (id >= 0 && id < a.num_pictures) {
      bool live = false;   // some binding has a non-neutral gain for this picture
#pragma unroll
      for (int j = 0; j < kMaxBindings; ++j) live |= j < a.nbind && a.lg2gain[j][id] != 0.0f;
      if (live) kp = id;
    }
  }
  const int64_t ki = (int64_t)b * a.npad + n;
  a.tk[ki] = tk;
  a.kp[ki] = kp;

  // tile summary
  const bool isp = kp >= 0;
  const bool all_plain = !wave_any(isg || isp);
  const bool all_guide = !wave_any(!isg);
  const int kp0 = __shfl(kp, 0);
  // one bound picture: the bias of a row is its gain-table entry
  const bool all_pic = !wave_any(!isp || kp != kp0);
  const bool any_pic = wave_any(isp);
  float lo = isg ? tk : INFINITY, hi = isg ? tk : -INFINITY;
  for (int off = 32; off >= 1; off >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, off));
    hi = fmaxf(hi, __shfl_xor(hi, off));
  }
  if (threadIdx.x == 0) {
    KeyTileSummary s;
    s.kind = (all_plain ? KT_PLAIN : all_guide ? KT_GUIDE : all_pic ? KT_PICTURE : KT_MIXED) |
             (any_pic ? KT_HAS_PICTURE : 0);
    s.lo = lo;
    s.hi = hi;
    s.pic = all_pic ? kp0 : -1;
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
// row N-1, as the attention kernel's staging does). 256 threads per tile; each
// wave reads 16 rows, four per load instruction: lane l takes 16 bytes of row
// l / (D/8) at chunk l % (D/8), so one instruction reads whole rows
// contiguously. A row's sum of squares is combined across its D/8 lanes, then
// the max is taken over the rows.
__global__ __launch_bounds__(256) void knorm_kernel(const __bf16* __restrict__ k, int64_t sb, int64_t sh, int64_t sn,
                                                    int H, int N, int D, int nkt, float* __restrict__ kmax) {
  __shared__ float wmax[4];
  const int t = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int cpr = D / 8;                 // 16-byte chunks per row (16 or 8)
  const int rpi = 64 / cpr;              // rows per load instruction (4 or 8)
  const int rpw = kBlockK / 4;           // rows per wave (16)
  const __bf16* kb = k + b * sb + h * sh;
  float m = 0.0f;
  for (int r0 = 0; r0 < rpw; r0 += rpi) {
    const int n = min(t * kBlockK + wave * rpw + r0 + lane / cpr, N - 1);
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(kb + (int64_t)n * sn + (lane % cpr) * 8);
    float ss = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float f = (float)v[e];
      ss = fmaf(f, f, ss);
    }
    for (int off = 1; off < cpr; off <<= 1) ss += __shfl_xor(ss, off);
    m = fmaxf(m, sqrtf(ss));
  }
  for (int off = cpr; off < 64; off <<= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (lane == 0) wmax[wave] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    // a norm past the fp32 range is held at FLT_MAX, so that the attention
    // kernel's bound |q| max|k| never becomes 0 * inf
    kmax[(int64_t)bh * nkt + t] = fminf(fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3])), FLT_MAX);
}

hipError_t launch_knorm(const __bf16* k, int64_t sb, int64_t sh, int64_t sn, float* kmax, int B, int H, int N,
                        int nkt, int D, hipStream_t s) {
  dim3 grid(nkt, B * H);
  hipLaunchKernelGGL(knorm_kernel, grid, dim3(256), 0, s, k, sb, sh, sn, H, N, D, nkt, kmax);
  return hipGetLastError();
}

// ------------------------------------------------- 8-bit Q.K: K quantisation
// FP8 E4M3 (OCP; round to nearest even, as v_cvt_pk_fp8_f32 does) with a
// power-of-two scale per 64-key tile of a head, 2^(floor(log2 max|k|) - 7),
// so the tile's largest magnitude lands in [128, 256). Writes
//   k8[b*H + h][n][d]  the scaled, rounded keys (rows past N are 0),
//   ks[b*H + h][t]     the tile's scale,
//   kmax[b*H + h][t]   max |k| over the tile's rounded rows (E4M3 codes times
//                      the scale), so that |q||k| bounds the 8-bit products.
// 256 threads per tile: four adjacent threads per row, D/4 elements each.

// floor(log2 |x|) of a finite x != 0 (exact, subnormals included)
__device__ __forceinline__ int floor_log2(float x) {
  int e;
  (void)frexpf(x, &e);
  return e - 1;
}

// Packs four floats (already scaled to |x| < 256) into four E4M3 bytes.
__device__ __forceinline__ uint32_t pack_fp8x4(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// Sum of the squares of four E4M3 codes (the values pack_fp8x4 rounded to), in
// fp32: the squares are exact, the sum rounds far inside the 2^-10 slack of the
// attention kernel's norm bound.
__device__ __forceinline__ float fp8x4_sumsq(uint32_t w) {
  const float a = __builtin_amdgcn_cvt_f32_fp8((int)w, 0), b = __builtin_amdgcn_cvt_f32_fp8((int)w, 1);
  const float c = __builtin_amdgcn_cvt_f32_fp8((int)w, 2), d = __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
  return fmaf(a, a, fmaf(b, b, fmaf(c, c, d * d)));
}

__global__ __launch_bounds__(256) void kquant_kernel(const __bf16* __restrict__ k, int64_t sb, int64_t sh, int64_t sn,
                                                     int H, int N, int D, int npad, int nkt, uint8_t* __restrict__ k8,
                                                     float* __restrict__ ks, float* __restrict__ kmax) {
  __shared__ float wred[2][4];
  const int t = blockIdx.x, bh = blockIdx.y, b = bh / H, h = bh % H;
  const int r = threadIdx.x >> 2, qd = threadIdx.x & 3;
  const int n = t * kBlockK + r;
  const bool valid = n < N;
  const int dq = D / 4;
  const __bf16* kp = k + b * sb + h * sh + (int64_t)(valid ? n : 0) * sn + qd * dq;
  float v[32];
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; i += 8) {
    if (i < dq) {
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(kp + i);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float f = valid ? (float)x[e] : 0.0f;
        v[i + e] = f;
        am = fmaxf(am, fabsf(f));
      }
    }
  }
  for (int off = 32; off >= 1; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
  if ((threadIdx.x & 63) == 0) wred[0][threadIdx.x >> 6] = am;
  __syncthreads();
  am = fmaxf(fmaxf(wred[0][0], wred[0][1]), fmaxf(wred[0][2], wred[0][3]));
  const int e = am > 0.0f ? floor_log2(am) - 7 : 0;   // scale 2^e
  uint8_t* dst = k8 + ((int64_t)bh * npad + n) * D + qd * dq;
  float ss = 0.0f;   // sum of squares of the row's E4M3 codes (this thread's share)
#pragma unroll
  for (int i = 0; i < 32; i += 16) {
    if (i < dq) {
      u32x4 w;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        w[j] = pack_fp8x4(ldexpf(v[i + 4 * j], -e), ldexpf(v[i + 4 * j + 1], -e), ldexpf(v[i + 4 * j + 2], -e),
                          ldexpf(v[i + 4 * j + 3], -e));
        ss += fp8x4_sumsq(w[j]);
      }
      *reinterpret_cast<u32x4*>(dst + i) = w;
    }
  }
  ss += __shfl_xor(ss, 1);
  ss += __shfl_xor(ss, 2);
  float nm = sqrtf(ss);   // the rounded row's norm over 2^e
  for (int off = 32; off >= 1; off >>= 1) nm = fmaxf(nm, __shfl_xor(nm, off));
  if ((threadIdx.x & 63) == 0) wred[1][threadIdx.x >> 6] = nm;
  __syncthreads();
  nm = fmaxf(fmaxf(wred[1][0], wred[1][1]), fmaxf(wred[1][2], wred[1][3]));
  if (threadIdx.x == 0) {
    ks[(int64_t)bh * nkt + t] = ldexpf(1.0f, e);
    kmax[(int64_t)bh * nkt + t] = fminf(ldexpf(nm, e), FLT_MAX);   // as in knorm_kernel
  }
}

hipError_t launch_kquant(const __bf16* k, int64_t sb, int64_t sh, int64_t sn, uint8_t* k8, float* ks, float* kmax,
                         int B, int H, int N, int npad, int nkt, int D, hipStream_t s) {
  dim3 grid(nkt, B * H);
  hipLaunchKernelGGL(kquant_kernel, grid, dim3(256), 0, s, k, sb, sh, sn, H, N, D, npad, nkt, k8, ks, kmax);
  return hipGetLastError();
}

// --------------------------------------------------------- bf16 MFMA kernel
// One workgroup = NW waves x 32 query rows of one (batch, head). Per 64-key
// tile t every wave runs a two-phase software pipeline so that its MFMAs and
// its softmax VALU work interleave in program order (MFMA and VALU of one wave
// co-issue; in-order issue means the VALU work has to sit between the MFMAs):
//   phase A: S_{t+1} = K_{t+1} Q^T (16 MFMAs)   with   P_t = exp2(X_t) and its bf16 pack
//   phase B: O^T += V_t^T P_t^T (16 MFMAs)      with   row sums of P_t, X_{t+1} = S_{t+1} c + b - m
// K runs one tile ahead of V. One ring of LDS fragment registers is fetched
// three fragments ahead through both phases and across iterations (the tail
// of phase A fetches V_t, the tail of phase B fetches K_{t+2}), so no LDS
// latency is exposed where a phase starts. Between the phases every wave
// waits for its own DMAs of K_{t+2} and V_{t+1}, and the workgroup meets at
// its one barrier per tile.

// Row pitch (floats) of the gain table copy in LDS: 16 pictures + 1 pad.
constexpr int kGtPitch = kMaxPictures + 1;

// LDS ring depth of the bf16 kernel (K and V^T tiles).
constexpr int kStages = 3;
// Key-loop start offset between consecutive query blocks, in key tiles
// (measured: 4 halves the L2 misses of lockstep starts; 2, 3, 5, 6 and 8 do
// less well).
constexpr int kRotTiles = 4;

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

// Chunk swizzle of the V^T tile in LDS: the 16-byte chunk c of V^T row r (8
// chunks of a 64-key row, no padding) sits at position c ^ vswz(r). The 16
// lanes of a fragment read that take rows r0 .. r0 + 15 (same chunk) then hit
// 16 different 16-byte bank groups: row r's bytes start at bank group
// 8 * (r & 1), and vswz covers (r >> 1) & 7.
__device__ __forceinline__ int vswz(int r) { return (r >> 1) & 7; }

// Tile staging by LDS DMA (buffer_load_dwordx4 ... lds): one wave instruction
// writes 64 lanes x 16 bytes contiguously at a uniform LDS address. A padded
// tile of BLK whole 1-KB blocks (rows of ROWB bytes holding DATA 16-byte data
// chunks) is staged by all NW waves: wave w takes blocks w, w + NW, ...
// (PER_MAX DMAs for waves w < BLK % NW, PER_MIN, possibly 0, for the others).
// A lane whose 16 bytes fall on a row's pad chunk re-reads chunk 0 of its row
// (never read back; masking those lanes off costs more in branches than the
// bytes save). Buffer loads rather than global_load_lds: the latter is
// FLAT-encoded, and while one is in flight the compiler cannot count LDS
// reads, so every fragment wait would drain all of them.
template <int ROWB, int DATA, int BLK, int NW, bool SWZ = false>
struct TileDma {
  static constexpr int PER_MIN = BLK / NW;
  static constexpr int PER_MAX = (BLK + NW - 1) / NW;
  static constexpr int NEXTRA = BLK % NW;
  static_assert(PER_MAX >= 1, "a tile is at least one block");
  uint32_t voff[PER_MAX];   // byte offset of this lane's 16 bytes in its tile
  int row[PER_MAX];         // tile row of those bytes
  __device__ void init(int wave, int lane, uint32_t row_bytes) {
#pragma unroll
    for (int p = 0; p < PER_MAX; ++p) {
      const int ci = min(wave + p * NW, BLK - 1);
      const int o = ci * 1024 + lane * 16, r = o / ROWB, c = (o % ROWB) / 16;
      row[p] = r;
      // SWZ: LDS chunk c of row r holds the row's chunk c ^ vswz(r)
      voff[p] = r * row_bytes + (SWZ ? (c ^ vswz(r)) * 16 : c < DATA ? c * 16 : 0);
    }
  }
  // Stage the tile at byte offset soff of r into lds (wave in [0, NW)). With
  // TAIL, rows at or past rows_left re-read row rows_left - 1 (their keys are
  // masked later).
  template <bool TAIL>
  __device__ void issue(BufRange r, uint32_t soff, int rows_left, uint32_t row_bytes, char* lds, int wave) const {
#pragma unroll
    for (int p = 0; p < PER_MAX; ++p) {
      if (p >= PER_MIN && wave >= NEXTRA) break;
      uint32_t vo = voff[p];
      if (TAIL) vo -= (uint32_t)(row[p] - min(row[p], rows_left - 1)) * row_bytes;
      dma16(r, vo, soff, lds + (wave + p * NW) * 1024);
    }
  }
};

// The bf16 K tile at head dim 128 without row padding: 16 blocks of 4 rows (1 KB
// each, one DMA each: exactly two per wave of eight), block b at LDS byte
// b * kKBlkPitch (the last 64 bytes of each pitch are never written), and the
// 16-byte chunk c of row r at chunk position c ^ (r & 3). The 16 lanes of a
// fragment read take 16 consecutive rows at one chunk: their 16-byte bank
// groups (4 * block + position) mod 16 are all different.
constexpr int kKBlkPitch = 1024 + 64;
template <int NW>
struct KTileDmaBlk {
  static constexpr int BLK = 16;
  static constexpr int PER_MIN = BLK / NW;
  static constexpr int PER_MAX = (BLK + NW - 1) / NW;
  static constexpr int NEXTRA = BLK % NW;
  uint32_t voff[PER_MAX];   // byte offset of this lane's 16 bytes in its tile
  int row[PER_MAX];         // tile row of those bytes
  __device__ void init(int wave, int lane, uint32_t row_bytes) {
#pragma unroll
    for (int p = 0; p < PER_MAX; ++p) {
      const int b = min(wave + p * NW, BLK - 1);
      const int r = 4 * b + (lane >> 4), pos = lane & 15;
      row[p] = r;
      voff[p] = r * row_bytes + (pos ^ (r & 3)) * 16;
    }
  }
  // as TileDma::issue (TAIL: rows at or past rows_left re-read row rows_left - 1)
  template <bool TAIL>
  __device__ void issue(BufRange rg, uint32_t soff, int rows_left, uint32_t row_bytes, char* lds, int wave) const {
#pragma unroll
    for (int p = 0; p < PER_MAX; ++p) {
      if (p >= PER_MIN && wave >= NEXTRA) break;
      uint32_t vo = voff[p];
      if (TAIL) vo -= (uint32_t)(row[p] - min(row[p], rows_left - 1)) * row_bytes;
      dma16(rg, vo, soff, lds + (wave + p * NW) * kKBlkPitch);
    }
  }
};

// Wait until at most KEEP of this wave's vector-memory operations are pending
// (the newest KEEP DMAs may stay in flight).
template <int KEEP>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(KEEP) : "memory");
}

// i-th K fragment of phase A: key block i & 1, head-dim step kk = i >> 1, from
// the K tile at kbuf; KBS is the element distance between the two 32-row key
// blocks. With two offsets, kl[kk & 1] is the lane's element offset for even /
// odd steps (they differ in the block layout of KTileDmaBlk) and step kk adds
// 16 elements; with one offset per step (swizzled 128-byte rows), kl[kk].
template <int KBS, int NKL>
__device__ __forceinline__ bf16x8 kfrag(const __bf16* kbuf, const int (&kl)[NKL], int i) {
  const int kk = i >> 1;
  int off;
  if constexpr (NKL == 2) off = kl[kk & 1] + kk * 16;
  else off = kl[kk];
  return *reinterpret_cast<const bf16x8*>(kbuf + (i & 1) * KBS + off);
}

// S^T for the two 32-key blocks of a K tile in LDS.
template <int D, int KBS, int NKL>
__device__ __forceinline__ void qk_tile(f32x16 (&s)[2], const __bf16* kbuf, const int (&kl)[NKL],
                                        const bf16x8 (&qf)[D / 16]) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    s[kb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag<KBS>(kbuf, kl, 2 * kk + kb), qf[kk], s[kb], 0, 0, 0);
  }
}

// i-th V^T fragment of phase B: 32-row block i % NDB of the head dim, 16-key
// chunk i / NDB (key block kb = chunk / 2, half c2 = chunk % 2). vr0 is the
// lane's row (db = 0) and vck[chunk] the element offset of its 16 bytes of
// that chunk in the swizzled row.
template <int VROW, int NDB>
__device__ __forceinline__ bf16x8 vfrag(const __bf16* vr0, const int (&vck)[4], int i) {
  return *reinterpret_cast<const bf16x8*>(vr0 + (i % NDB) * 32 * VROW + vck[i / NDB]);
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// 8-bit Q.K: S^T (32 keys x 32 queries) += K8 (32 keys x 64 dims, FP8 E4M3)
// x Q8^T with fp32 accumulation (v_mfma_scale_f32_32x32x64_f8f6f4, block
// scales 1.0). Operand layout: lane l holds row (A) / column (B) l % 32 and the
// 32 consecutive dims 32*(l/32) .. +31 of the 64.
__device__ __forceinline__ f32x16 mfma_fp8(i32x8 k8, i32x8 q8, f32x16 acc) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(k8, q8, acc, 0, 0, 0, 127, 0, 127);
}

// i-th fp8 K fragment of phase A: key block i & 1, 64-dim step i >> 1: the
// lane's 32 bytes of its K row (kr0: the row in key block 0, LDS row pitch
// KROWB bytes), two 16-byte chunks at the byte offsets k8o[2 * step] and
// k8o[2 * step + 1] within the row (swizzled rows place the chunks apart).
template <int KROWB>
__device__ __forceinline__ i32x8 kfrag8(const char* kr0, const int (&k8o)[4], int i) {
  const char* p = kr0 + (i & 1) * 32 * KROWB;
  const u32x4 lo = *reinterpret_cast<const u32x4*>(p + k8o[2 * (i >> 1)]);
  const u32x4 hi = *reinterpret_cast<const u32x4*>(p + k8o[2 * (i >> 1) + 1]);
  i32x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
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
  r.pic = p[i].pic;
  return r;
}

// Bias class of one key tile for one query row: returns true when the tile
// needs the per-element formula for this row; otherwise *brow is the row's
// constant bias over the tile (log2 units; -inf: the tile adds nothing to this
// row's pass).
template <int PASS>
__device__ __forceinline__ bool tile_class_lane(const KeyTileSummary& sm, bool partial, bool qbiased, float tq,
                                                float gpic, const AttnArgs& a, float* brow) {
  float b = 0.0f;
  bool lane_elem = partial;
  if (!partial) {
    const int kind = sm.kind & KT_CLASS;
    const float dlo = sm.lo - tq, dhi = tq - sm.hi;
    const float dmin = fmaxf(fmaxf(dlo, dhi), 0.0f);
    const float dmax = fmaxf(-dlo, -dhi);
    if (PASS == PASS_TERM_A) {
      // keys that are not biased guide keys, normal logits
      if (kind == KT_GUIDE) b = -INFINITY;
      else if (kind == KT_PICTURE) b = gpic;
      else if (kind == KT_MIXED) lane_elem = true;
    } else if (PASS == PASS_TERM_B) {
      // biased guide keys, target rows at -cap
      if (kind == KT_GUIDE) b = qbiased ? -a.cap2 : 0.0f;
      else if (kind == KT_MIXED) lane_elem = true;
      else b = -INFINITY;
    } else if (PASS == PASS_TERM_C) {
      // biased guide keys x target rows: s + log2(2^-penalty - 2^-cap)
      if (kind == KT_GUIDE && qbiased) {
        if (dmin >= a.dsat) b = -INFINITY;
        else if (dmax <= a.window) b = a.corr0;
        else lane_elem = true;
      } else if (kind == KT_MIXED && qbiased) {
        lane_elem = true;
      } else {
        b = -INFINITY;
      }
    } else {
      if (kind == KT_GUIDE) {
        if (qbiased) {
          if (dmin >= a.dsat) b = -a.cap2;
          else if (!(dmax <= a.window)) lane_elem = true;
        }
      } else if (kind == KT_PICTURE) {
        b = gpic;
      } else if (kind == KT_MIXED) {
        lane_elem = true;
      }
    }
  }
  *brow = b;
  return lane_elem;
}

// Per-element logits of a key tile, in place (log2 units), keys outside
// [k0, k1) -> -inf; cmul turns a raw product into log2 units (the softmax
// scale times log2 e, times the fp8 scales for 8-bit Q.K). Fused / range
// passes: x = s*cmul - penalty + binding, where
// binding is the query's summed log2 gain of the key's picture (gtq: this row
// of the gain table, in LDS; read only when the tile holds bound picture
// keys). Term passes keep only their keys (see PASS_TERM_*). A key is a biased
// guide key when its encoded time is not NaN. Lane half hh holds keys
// 8*hh..8*hh+7 and 16+8*hh..16+8*hh+7 of each 32-key block.
template <int PASS>
__device__ __forceinline__ void elem_bias(f32x16 (&s)[2], int kbase, int hh, float tq, bool has_pic,
                                          const float* gtq, bool partial, int k0, int k1, const float* tkb,
                                          const int* kpb, const AttnArgs& a, float cmul) {
  const bool qb = tq == tq;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int c2 = 0; c2 < 2; ++c2) {
      const int kx = kbase + kb * 32 + c2 * 16 + hh * 8;
      const f32x4 t0 = *reinterpret_cast<const f32x4*>(tkb + kx);
      const f32x4 t1 = *reinterpret_cast<const f32x4*>(tkb + kx + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float tk = e < 4 ? t0[e] : t1[e - 4];
        const float dd = fmaxf(fmaf(fabsf(tq - tk), a.sigma, -a.w), 0.0f);   // NaN time -> 0
        const float pen = fminf(dd * dd, a.cap2);
        const float sv = s[kb][c2 * 8 + e];
        const bool isg = tk == tk;
        float x;
        if (PASS == PASS_TERM_A) x = isg ? -INFINITY : sv * cmul;
        else if (PASS == PASS_TERM_B) x = isg ? fmaf(sv, cmul, qb ? -a.cap2 : 0.0f) : -INFINITY;
        else if (PASS == PASS_TERM_C)
          x = isg && qb ? fmaf(sv, cmul, __log2f(1.0f - fast_exp2(pen - a.cap2)) - pen) : -INFINITY;
        else x = fmaf(sv, cmul, -pen);
        s[kb][c2 * 8 + e] = x;
      }
    }
  }
  if (has_pic && (PASS == PASS_FUSED || PASS == PASS_RANGE || PASS == PASS_TERM_A)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int c4 = 0; c4 < 4; ++c4) {
        const int kx = kbase + kb * 32 + (c4 >> 1) * 16 + hh * 8 + (c4 & 1) * 4;
        const int4 pk = *reinterpret_cast<const int4*>(kpb + kx);
        const int pe[4] = {pk.x, pk.y, pk.z, pk.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (pe[e] >= 0) s[kb][c4 * 4 + e] += gtq[pe[e]];
      }
  }
  if (partial) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kbase + kb * 32 + (r >> 3) * 16 + hh * 8 + (r & 7);
        if (key < k0 || key >= k1) s[kb][r] = -INFINITY;
      }
  }
}

template <int V>
struct SlotIndex {
  static constexpr int value = V;
};

template <int D, int NW, int PASS, bool Q8, bool DB>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4)))
void attn_bf16_kernel(AttnArgs a) {
  constexpr bool PART = PASS != PASS_FUSED;   // writes one partition's (O_p, LSE_p)
  constexpr bool TERM = PASS >= PASS_TERM_A;  // visits a listed subset of the key tiles
  static_assert(!Q8 || PASS == PASS_FUSED || PASS == PASS_RANGE,
                "8-bit Q.K is built for the fused pass and the range pass of a fused call's tail");
  // DB: the dense-bias baseline reads every logit's bias from a.dbias instead
  // of computing it
  static_assert(!DB || (PASS == PASS_FUSED && !Q8), "the dense-bias baseline is a fused bf16 pass");
  constexpr int BQ = NW * 32;              // query rows per workgroup
  // bf16 K rows at D = 64: 128 bytes, 16-byte chunks swizzled like V^T rows
  // (vswz), no padding; at D = 128 see KBLK below
  constexpr bool K64SWZ = !Q8 && D == 64;
  constexpr int KROW = K64SWZ ? D : D + 8;  // LDS pitch of a bf16 K row (elements)
  // LDS pitch of a K row in bytes (FP8 rows: D bytes + a 16-byte pad)
  // FP8 K rows at D = 128: 128 bytes, 16-byte chunks swizzled like V^T rows
  // (vswz), no padding; at D = 64 padded by 16 bytes
  constexpr bool K8SWZ = Q8 && D == 128;
  constexpr int KROWB = Q8 ? (K8SWZ ? D : D + 16) : KROW * 2;
  // bf16 K at D = 128: unpadded rows in blocks (KTileDmaBlk); the same tile size
  constexpr bool KBLK = !Q8 && D == 128;
  static_assert(!KBLK || 16 * kKBlkPitch == kBlockK * KROW * 2, "the block layout keeps the tile size");
  constexpr int KBS = KBLK ? 8 * kKBlkPitch / 2 : 32 * KROW;   // elements between the two 32-row key blocks
  // V^T rows in LDS: swizzled 16-byte chunks without padding (vswz), except in
  // the dense-bias baseline, whose bias loads leave no registers for the four
  // per-lane chunk offsets the swizzle needs: there rows are padded by 16 bytes
  constexpr bool VSWZ = !DB;
  constexpr int VROW = VSWZ ? kBlockK : kBlockK + 8;   // LDS pitch of a V^T row (elements)
  constexpr int KTILE = kBlockK * KROWB / 2;   // K tile size in bf16 elements
  constexpr int VTILE = D * VROW;
  constexpr int NKK = D / 16;
  constexpr int NDB = D / 32;
  constexpr int NA = Q8 ? 2 * (D / 64) : 2 * NKK;   // MFMAs of phase A (K fragments)
  constexpr int NB = 4 * NDB;              // MFMAs (and LDS fragments) of phase B
  static_assert((Q8 || NA % 4 == 0) && NB % 4 == 0, "ring positions carry over between the phases");
  // LDS ring of NS stages: K tiles in slots 0..NS-1, then V^T tiles in slots 0..NS-1
  constexpr int NS = kStages;
  static_assert(NS == 3, "slot arithmetic and the DMA wait count assume three stages");
  // one LDS array (the K/V^T ring, then the workgroup's rows of the gain
  // table with row pitch kGtPitch floats, then for term passes the list of
  // key tiles to visit and a little scratch): with a second array the
  // compiler can no longer tell the ring's DMA writes from other LDS reads and
  // waits for every DMA before each fragment read
  constexpr int GT_ELEMS = BQ * kGtPitch * 2;
  constexpr int LIST_ELEMS = TERM ? kMaxListTiles + 4 * NW : 0;
  __shared__ __attribute__((aligned(16))) __bf16 smem[NS * (KTILE + VTILE) + GT_ELEMS + LIST_ELEMS];
  float* const gt_lds = reinterpret_cast<float*>(smem + NS * (KTILE + VTILE));
  uint16_t* const tlist = reinterpret_cast<uint16_t*>(smem + NS * (KTILE + VTILE) + GT_ELEMS);
  int* const tscr = reinterpret_cast<int*>(tlist + kMaxListTiles);   // 2*NW ints
#define KBUF(i) (smem + (i) * KTILE)
#define VBUF(i) (smem + NS * KTILE + (i) * VTILE)

  const int part = PASS == PASS_RANGE ? blockIdx.y : TERM ? PASS - PASS_TERM_A : 0;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = L / a.nqb, qblk = L % a.nqb;
  const int b = bh / a.H, h = bh % a.H;
  const int N = a.N;

  const int tid = threadIdx.x, lane = tid & 63, lq = lane & 31, hh = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6) & (NW - 1);   // uniform per wave

  // this lane's query row: column lq of the wave's S^T blocks
  const int qrow = a.qr0 + qblk * BQ + wave * 32 + lq;   // rows [qr0, qr1) of this launch
  const bool qvalid = qrow < a.qr1;
  const int qr = qvalid ? qrow : a.qr1 - 1;
  bf16x8 qf[Q8 ? 1 : NKK];
  i32x8 qf8[Q8 ? D / 64 : 1];
  float q_ss = 0.0f;                       // |q|^2 of the lane's share of the row
  float cq = a.c;                          // 8-bit Q.K: softmax scale * log2 e * the row's scale
  {
    const __bf16* qp = static_cast<const __bf16*>(a.q) + b * a.q_sb + h * a.q_sh + (int64_t)qr * a.q_sn;
    if constexpr (!Q8) {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qp + kk * 16 + hh * 8);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) q_ss = fmaf((float)qf[kk][e], (float)qf[kk][e], q_ss);
    } else {
      // FP8 E4M3 with the row's power-of-two scale 2^(floor(log2 max|q|) - 7);
      // this lane holds dims 64*st + 32*hh .. +31 of each 64-dim step st
      float qv[D / 2];
      float am = 0.0f;
#pragma unroll
      for (int st = 0; st < D / 64; ++st)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bf16x8 x8 = *reinterpret_cast<const bf16x8*>(qp + st * 64 + hh * 32 + u * 8);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float f = (float)x8[e];
            qv[st * 32 + u * 8 + e] = f;
            am = fmaxf(am, fabsf(f));
          }
        }
      am = xor32_max(am);
      const int e = am > 0.0f ? floor_log2(am) - 7 : 0;
      cq = a.c * ldexpf(1.0f, e);
#pragma unroll
      for (int st = 0; st < D / 64; ++st)
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          qf8[st][w] = (int)pack_fp8x4(ldexpf(qv[st * 32 + w * 4], -e), ldexpf(qv[st * 32 + w * 4 + 1], -e),
                                       ldexpf(qv[st * 32 + w * 4 + 2], -e), ldexpf(qv[st * 32 + w * 4 + 3], -e));
          q_ss += fp8x4_sumsq((uint32_t)qf8[st][w]);   // |q|^2 of the rounded row over 2^(2e)
        }
    }
  }
  const float tq = a.tq[(int64_t)b * N + qr];
  const bool qbiased = tq == tq;
  // this row of the gain table into LDS (entry 0 is 0 when there is no table)
  const float* gtq = gt_lds + (wave * 32 + lq) * kGtPitch;
  if (hh == 0) {
    const float* g = a.gt + ((int64_t)b * N + qr) * a.npics;
    for (int p = 0; p < (a.npics > 0 ? a.npics : 1); ++p)
      gt_lds[(wave * 32 + lq) * kGtPitch + p] = p < a.npics ? g[p] : 0.0f;
  }

  const int k0 = TERM ? 0 : a.kr[part], k1 = TERM ? N : a.kr[part + 1];
  // an empty partition contributes nothing to the merge
  auto write_empty = [&]() {
    if (PART && qvalid) {
      float* op = a.opart + ((((int64_t)part * a.B + b) * a.H + h) * a.prows + (qrow - a.prow0)) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) *reinterpret_cast<f32x4*>(op + db * 32 + j * 8 + hh * 4) = f32x4{};
      if (hh == 0) a.lsepart[(((int64_t)part * a.B + b) * a.H + h) * a.prows + (qrow - a.prow0)] = -INFINITY;
    }
  };
  if (k1 <= k0) {
    write_empty();
    return;
  }
  const int kt0 = k0 / kBlockK, kt1 = (k1 + kBlockK - 1) / kBlockK;

  // tiles this pass visits: kt0 .. kt1-1, or for a term pass the listed ones
  int ntiles = kt1 - kt0;
  if (TERM) {
    // times of this workgroup's biased rows
    float tlo = qbiased && qvalid ? tq : INFINITY, thi = qbiased && qvalid ? tq : -INFINITY;
    for (int off = 32; off >= 1; off >>= 1) {
      tlo = fminf(tlo, __shfl_xor(tlo, off));
      thi = fmaxf(thi, __shfl_xor(thi, off));
    }
    float* tsf = reinterpret_cast<float*>(tscr);
    if (lane == 0) {
      tsf[wave] = tlo;
      tsf[NW + wave] = thi;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      tlo = fminf(tlo, tsf[w]);
      thi = fmaxf(thi, tsf[NW + w]);
    }
    __syncthreads();
    // compact the indices of the tiles holding keys of this term
    const KeyTileSummary* ks_g = a.ksum + (int64_t)b * a.nkt;
    int base = 0;
    for (int r = 0; r < a.nkt; r += NW * 64) {
      const int i = r + tid;
      bool keep = false;
      if (i < a.nkt) {
        const KeyTileSummary sm = ks_g[i];
        const bool has_guide = sm.lo <= sm.hi;   // some biased guide key
        if (PASS == PASS_TERM_A) keep = (sm.kind & KT_CLASS) != KT_GUIDE;
        else if (PASS == PASS_TERM_B) keep = has_guide;
        else keep = has_guide && tlo <= thi && fmaxf(fmaxf(sm.lo - thi, tlo - sm.hi), 0.0f) < a.dsat;
      }
      const uint64_t bal = __builtin_amdgcn_ballot_w64(keep);
      const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
      if (lane == 0) tscr[wave] = __builtin_popcountll(bal);
      __syncthreads();
      int off = base, tot = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int c = tscr[w];
        off += w < wave ? c : 0;
        tot += c;
      }
      if (keep) tlist[off + below] = (uint16_t)i;
      __syncthreads();
      base += tot;
    }
    ntiles = __builtin_amdgcn_readfirstlane(base);   // the same for every wave
    if (ntiles == 0) {
      write_empty();
      return;
    }
  }
  // key tile visited at step i (steps past the end repeat the last tile: the
  // ring slot it is staged into is free either way). The workgroups sharing an
  // XCD's L2 run consecutive query blocks and stream the same K/V^T tiles; in
  // lockstep they would all miss on a tile together, so each starts its loop
  // kRotTiles tiles after the previous query block's (within 32 blocks): the
  // first to reach a tile fetches it and the ones behind hit in L2. Any key
  // order gives the same softmax; the rotation is fixed per query block, so
  // results stay reproducible.
  const int krot = (qblk & 31) * kRotTiles % ntiles;
  // position in the pass's tile sequence (kt0 .. kt1-1, or the term list) of step i
  auto step_pos = [&](int i) -> int {
    const int j = min(i, ntiles - 1) + krot;
    return j >= ntiles ? j - ntiles : j;
  };
  auto tile_at = [&](int i) -> int {
    if (TERM) return __builtin_amdgcn_readfirstlane((int)tlist[step_pos(i)]);
    return kt0 + step_pos(i);
  };

  // staging: buffer ranges over this head's K rows and V^T rows; per-lane
  // 32-bit offsets within a tile, per-tile scalar offsets
  // (8-bit Q.K stages the FP8 copy of K, rows of D bytes, zero past N)
  const void* kg = Q8 ? static_cast<const void*>(a.k8 + (int64_t)bh * a.npad * D)
                      : static_cast<const void*>(static_cast<const __bf16*>(a.k) + b * a.k_sb + h * a.k_sh);
  const __bf16* vg = a.vt + (int64_t)bh * D * a.npad;
  const uint32_t k_sn_bytes = Q8 ? (uint32_t)D : (uint32_t)(a.k_sn * 2);
  const BufRange rk{kg, Q8 ? (uint32_t)(a.npad * D) : (uint32_t)(N - 1) * k_sn_bytes + D * 2};
  const BufRange rv{vg, (uint32_t)(D * a.npad * 2)};
  static_assert(KTILE * 2 % 1024 == 0 && VTILE * 2 % 1024 == 0, "tiles are whole 1-KB blocks");
  using KDma = std::conditional_t<KBLK, KTileDmaBlk<NW>, TileDma<KROWB, Q8 ? D / 16 : D / 8, KTILE * 2 / 1024, NW, K8SWZ || K64SWZ>>;
  using VDma = TileDma<VROW * 2, kBlockK / 8, VTILE * 2 / 1024, NW, VSWZ>;
  KDma kdma;
  VDma vdma;
  kdma.init(wave, lane, k_sn_bytes);
  vdma.init(wave, lane, (uint32_t)a.npad * 2);
  // K tile kk into K slot sk, V^T tile kv into V slot sv
  auto stage_k = [&](int kk, int sk) {
    const int rows_left = N - kk * kBlockK;
    const uint32_t soff = (uint32_t)kk * kBlockK * k_sn_bytes;
    char* l = reinterpret_cast<char*>(KBUF(sk));
    if (Q8 || rows_left >= kBlockK) kdma.template issue<false>(rk, soff, rows_left, k_sn_bytes, l, wave);
    else kdma.template issue<true>(rk, soff, rows_left, k_sn_bytes, l, wave);
  };
  auto stage_v = [&](int kv, int sv) {
    vdma.template issue<false>(rv, (uint32_t)kv * kBlockK * 2, kBlockK, 0, reinterpret_cast<char*>(VBUF(sv)), wave);
  };
  // this wave's DMAs of K_{t+2} and V_{t+1} have landed; those of K_{t+3},
  // issued after them, may stay in flight
  auto wait_staged = [&]() {
    if (wave < KDma::NEXTRA) wait_vm<KDma::PER_MAX>();
    else wait_vm<KDma::PER_MIN>();
  };

  const float* tkb = a.tk + (int64_t)b * a.npad;
  const int* kpb = a.kp + (int64_t)b * a.npad;
  // tile summaries and key norms through the constant address space: uniform
  // loads of them become scalar loads
  const KsumConstPtr ks_c = (KsumConstPtr)(a.ksum + (int64_t)b * a.nkt);
  const __attribute__((address_space(4))) float* kmax_c =
      (const __attribute__((address_space(4))) float*)(a.kmax + (int64_t)bh * a.nkt);
  // 8-bit Q.K: the key tiles' power-of-two scales
  const __attribute__((address_space(4))) float* kscale_c =
      (const __attribute__((address_space(4))) float*)(Q8 ? a.ks + (int64_t)bh * a.nkt : a.kmax);
  const int krow_lane = perm32(lq);
  // |q| * c, rounded up by 2^-10 to cover fp32 rounding of the MFMA sum; with
  // 8-bit Q.K, |q| and the key norms are those of the rounded values (E4M3
  // codes times their scales), so the bound covers the 8-bit products as tightly
  // (held at FLT_MAX like the key norms: the bound of a zero row against a
  // zero tile stays 0, the exact maximum, instead of 0 * inf)
  const float qn_c = fminf(sqrtf(xor32_sum(q_ss)) * (Q8 ? cq : a.c) * (1.0f + 0x1.0p-10f), FLT_MAX);

  f32x16 o[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) o[i] = f32x16{};
  float m_used, lsum = 0.0f;
  f32x16 x[2];   // X_t = S_t * c + bias - m_used (exp2 argument)
  KeyTileSummary sm_next;
  float kmax_next, kscale_next = 1.0f;
  // LDS fragment ring: fragment j of the per-wave stream (K_{t+1} fragments of
  // phase A, then V_t fragments of phase B, then K_{t+2} ...) sits in fr[j & 3];
  // with 8-bit Q.K the K fragments (32 bytes each) go through kf8 instead
  bf16x8 fr[4];
  i32x8 kf8[2];
  // phase A reads K rows kb*32 + perm32(lq): the lane's element offsets for even
  // and odd head-dim steps (equal unless KBLK: there row r's chunk 2*kk + hh sits
  // at position (2*kk + hh) ^ (r & 3), 16 elements later or earlier); with
  // K64SWZ one offset per step kk, chunk 2*kk + hh of row r at (2*kk + hh) ^ vswz(r)
  constexpr int NKL = K64SWZ ? NKK : 2;
  int kl[NKL];
  if constexpr (K64SWZ) {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) kl[kk] = krow_lane * KROW + ((2 * kk + hh) ^ vswz(krow_lane)) * 8;
  } else if constexpr (KBLK) {
    const int i_in = krow_lane & 3, b1 = i_in >> 1;
    const int base = (krow_lane >> 2) * (kKBlkPitch / 2) + i_in * D + 8 * (hh ^ (i_in & 1));
    kl[0] = base + 16 * b1;
    kl[1] = base - 16 * b1;
  } else {
    kl[0] = kl[1] = krow_lane * KROW + hh * 8;
  }
  const int koffb8 = krow_lane * KROWB;              // the same rows, FP8 bytes
  // byte offsets in that row of the lane's chunks 4 * step + 2 * hh + half
  int k8o[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int ch = 4 * (c >> 1) + 2 * hh + (c & 1);
    k8o[c] = (K8SWZ ? ch ^ vswz(krow_lane) : ch) * 16;
  }
  const int voff_lane = lq * VROW + (VSWZ ? 0 : hh * 8);   // phase B reads V^T rows db*32 + lq
  // element offsets of the lane's 16 bytes of 16-key chunk kc (keys 16*kc + 8*hh
  // .. +7) in its V^T row (swizzled: rows db*32 + lq share vswz, as 32 | db*32)
  int vck[4];
#pragma unroll
  for (int kc = 0; kc < 4; ++kc) vck[kc] = VSWZ ? ((2 * kc + hh) ^ vswz(lq)) * 8 : kc * 16;
  // raw Q.K products to log2 units for a tile (cq: the row part; times the tile's scale)
  auto tile_mul = [&](float kscale) { return Q8 ? cq * kscale : a.c; };
  // dense-bias baseline: this row of the bias tensor (pitch npad floats);
  // bv[kb*4 + c2*2 + u] holds keys kb*32 + c2*16 + 8*hh + 4*u .. +3 of a tile
  const float* dbq = DB ? a.dbias + ((int64_t)b * N + qr) * a.npad + 8 * hh : nullptr;
  auto load_dbias = [&](f32x4 (&bv)[8], int kbase) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      bv[i] = *reinterpret_cast<const f32x4*>(dbq + kbase + (i >> 2) * 32 + ((i >> 1) & 1) * 16 + (i & 1) * 4);
  };
  auto apply_dbias = [&](f32x16 (&sv)[2], const f32x4 (&bv)[8], float cmul) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sv[kb][r] = fmaf(sv[kb][r], cmul, bv[kb * 4 + (r >> 2)][r & 3]);
  };

  {
    // prologue: the first three tiles' K into K slots 0..2, the first two
    // tiles' V^T into V slots 0 and 1; S and X of the first tile; the first
    // three K fragments of the second tile
    const int tile0 = tile_at(0);
    stage_k(tile0, 0);
    stage_k(tile_at(1), 1);
    stage_k(tile_at(2), 2);
    stage_v(tile0, 0);
    stage_v(tile_at(1), 1);
    wait_vm<0>();
    __builtin_amdgcn_s_barrier();
    if constexpr (Q8) {
      const char* k8r = reinterpret_cast<const char*>(KBUF(0)) + koffb8;
      x[0] = x[1] = f32x16{};
#pragma unroll
      for (int i = 0; i < NA; ++i) x[i & 1] = mfma_fp8(kfrag8<KROWB>(k8r, k8o, i), qf8[i >> 1], x[i & 1]);
    } else {
      qk_tile<D, KBS>(x, KBUF(0), kl, qf);
    }
    const int kbase = tile0 * kBlockK;
    const bool partial = a.elem_all || kbase < k0 || kbase + kBlockK > k1;
    const KeyTileSummary sm0 = load_summary(ks_c, tile0);
    const float gpic0 = gtq[max(sm0.pic, 0)];
    float brow;
    const bool lane_elem = tile_class_lane<PASS>(sm0, partial, qbiased, tq, gpic0, a, &brow);
    float cc = tile_mul(Q8 ? kscale_c[tile0] : 1.0f);
    if constexpr (DB) {
      f32x4 bv0[8];
      load_dbias(bv0, kbase);
      apply_dbias(x, bv0, cc);
      brow = 0.0f;
      cc = 1.0f;
    } else if (wave_any(lane_elem)) {
      elem_bias<PASS>(x, kbase, hh, tq, (sm0.kind & KT_HAS_PICTURE) != 0, gtq, partial, k0, k1, tkb, kpb, a, cc);
      brow = 0.0f;
      cc = 1.0f;
    }
    float mx = x[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, x[kb][r]);
    // a row with no finite logit yet keeps m = -inf; its exponent reference is 0
    m_used = fmaf(xor32_max(mx), cc, brow);
    const float off = brow - (m_used == -INFINITY ? 0.0f : m_used);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[kb][r] = fmaf(x[kb][r], cc, off);
    sm_next = load_summary(ks_c, tile_at(1));
    kmax_next = kmax_c[tile_at(1)];
    if (Q8) kscale_next = kscale_c[tile_at(1)];
    if constexpr (Q8) {
      kf8[0] = kfrag8<KROWB>(reinterpret_cast<const char*>(KBUF(1)) + koffb8, k8o, 0);
    } else {
      const __bf16* kr0 = KBUF(1);
      fr[0] = kfrag<KBS>(kr0, kl, 0);
      fr[1] = kfrag<KBS>(kr0, kl, 1);
      fr[2] = kfrag<KBS>(kr0, kl, 2);
    }
    // every wave is done with K slot 0 before iteration t0 restages it
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::"s"(sm_next.kind), "s"(sm_next.lo), "s"(sm_next.hi), "s"(sm_next.pic), "s"(kmax_next),
                 "s"(kscale_next));
  }

  // ring slots at step t (visiting tile T_t): K and V^T of T_t in s0, of
  // T_{t+1} in s1; K of T_{t+2} and V^T of T_{t-1} in s2. K of T_{t+3} is
  // staged into s0 at the start (T_t's K was last read before the previous
  // barrier), V^T of T_{t+2} into s2 after this step's barrier (T_{t-1}'s V^T
  // was last read before it). tw1..tw3 hold T_{t+1} .. T_{t+3}; a term pass
  // reads T_{t+4} from its LDS list one step ahead (tv4).
  int tw1 = tile_at(1), tw2 = tile_at(2), tw3 = tile_at(3);
  // one step; the ring slots are compile-time constants (the loop below is
  // unrolled by NS), so the slot arithmetic folds into the LDS offsets
  auto step = [&](auto slot, int t) __attribute__((always_inline)) {
    constexpr int s0 = decltype(slot)::value;
    constexpr int s1 = (s0 + 1) % NS;
    constexpr int s2 = (s0 + 2) % NS;
    const bool has1 = t + 1 < ntiles;
    int tv4 = 0;
    if (TERM) tv4 = tlist[step_pos(t + 4)];
    const KeyTileSummary sm1 = sm_next;
    const float kmax1 = kmax_next;
    const float kscale1 = kscale_next;
    // a one-picture tile's bias is this row's gain-table entry for the
    // picture (read every tile, so no path waits on a pending load)
    const float gpic1 = gtq[max(sm1.pic, 0)];
    // dense-bias baseline: the bias of tile t+1, loaded before K_{t+3} is
    // staged so that waiting for it leaves that DMA in flight
    f32x4 bv1[8];
    if (DB && has1) load_dbias(bv1, tw1 * kBlockK);
    stage_k(tw3, s0);
    const int kbase1 = tw1 * kBlockK;
    const bool partial1 = a.elem_all || kbase1 < k0 || kbase1 + kBlockK > k1;
    // bias class of tile t+1, worked out before phase A (it needs only the
    // tile summary, the row and m, all known here): a per-row constant brow,
    // or the per-element path if some lane needs it (cls_elem); cls_bound:
    // every logit of the tile is <= |q| max|k| c + brow (Cauchy-Schwarz), and
    // the exact row max is needed only when that bound could pass m + tau
    float brow = 0.0f;
    bool cls_elem = false, cls_bound = false;
    if (!DB && has1) {
      const bool lane_elem = tile_class_lane<PASS>(sm1, partial1, qbiased, tq, gpic1, a, &brow);
      cls_elem = wave_any(lane_elem);
      cls_bound = wave_any(fmaf(qn_c, kmax1, brow) > m_used + kRescaleTau);
    }
    const __bf16* kr0 = KBUF(s1);   // K_{t+1}
    const __bf16* vr0 = VBUF(s0) + voff_lane;   // V_t
    const __bf16* kn0 = KBUF(s2);   // K_{t+2}

    // phase A: S_{t+1} = K_{t+1} Q^T (the two 32-key blocks alternate) |
    // P_t = exp2(X_t) in place and its bf16 pack. The ring runs three
    // fragments ahead; its last three fetches are phase B's first V_t fragments.
    f32x16 sn[2];
    sn[0] = sn[1] = f32x16{};
    u32x4 pw[4];   // P_t as packed bf16 pairs: pw[kb*2 + c2] is the B operand of PV chunk (kb, c2)
    // elements 2i, 2i+1 of the lane's 32 scores of tile t: exp2 in place,
    // then (one MFMA slot later, off the exp latency) the bf16 pack
    auto exp_only = [&](int i) {
      const int kb = i >> 3, r = (2 * i) & 15;
      x[kb][r] = fast_exp2(x[kb][r]);
      x[kb][r + 1] = fast_exp2(x[kb][r + 1]);
    };
    auto pack_pair = [&](int i) {
      const int kb = i >> 3, r = (2 * i) & 15;
      pw[i >> 2][i & 3] = pack_bf16x2(x[kb][r], x[kb][r + 1]);
    };
    auto exp_pair = [&](int i) {
      exp_only(i);
      pack_pair(i);
    };
    if constexpr (Q8) {
      // four (D 128) or two (D 64) FP8 products, the K fragments one ahead;
      // the V_t fragments for phase B are fetched under the last one
      const char* k8r = reinterpret_cast<const char*>(KBUF(s1)) + koffb8;
      constexpr int EPM = 16 / NA;
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        if (i + 1 < NA) {
          kf8[(i + 1) & 1] = kfrag8<KROWB>(k8r, k8o, i + 1);
        } else {
          fr[0] = vfrag<VROW, NDB>(vr0, vck, 0);
          fr[1] = vfrag<VROW, NDB>(vr0, vck, 1);
          fr[2] = vfrag<VROW, NDB>(vr0, vck, 2);
        }
        sn[i & 1] = mfma_fp8(kf8[i & 1], qf8[i >> 1], sn[i & 1]);
#pragma unroll
        for (int u = 0; u < EPM; ++u) exp_pair(i * EPM + u);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        const int j = i + 3;
        if (j < NA) fr[j & 3] = kfrag<KBS>(kr0, kl, j);
        else fr[j & 3] = vfrag<VROW, NDB>(vr0, vck, j - NA);
        sn[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i & 3], qf[i >> 1], sn[i & 1], 0, 0, 0);
        if (i < 16) exp_only(i);
        if (i >= 1 && i <= 16) pack_pair(i - 1);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = NA; i < 16; ++i) exp_only(i);
#pragma unroll
      for (int i = NA < 17 ? NA - 1 : 16; i < 16; ++i) pack_pair(i);
    }
    // keep P_t in this block (the PV product that reads it follows the
    // bias-class branch)
    asm volatile("" ::"v"(pw[0]), "v"(pw[1]), "v"(pw[2]), "v"(pw[3]));

    // the rare per-element bias path of tile t+1, before phase B
    float cc = tile_mul(kscale1);
    bool need_max = false;
    if (DB && has1) {
      apply_dbias(sn, bv1, cc);
      cc = 1.0f;
      need_max = true;
    } else if (has1) {
      if (cls_elem) {
        elem_bias<PASS>(sn, kbase1, hh, tq, (sm1.kind & KT_HAS_PICTURE) != 0, gtq, partial1, k0, k1, tkb, kpb,
                        a, cc);
        brow = 0.0f;
        cc = 1.0f;
        need_max = true;
      } else {
        need_max = cls_bound;
      }
    }
    float m_new = m_used;
    if (need_max) {
      float mxa = -INFINITY, mxb = -INFINITY;
#pragma unroll
      for (int f = 0; f < 32; f += 4) {
        mxa = max3f(mxa, sn[f >> 4][f & 15], sn[f >> 4][(f & 15) + 1]);
        mxb = max3f(mxb, sn[f >> 4][(f & 15) + 2], sn[f >> 4][(f & 15) + 3]);
      }
      const float mt = fmaf(xor32_max(fmaxf(mxa, mxb)), cc, brow);
      if (mt > m_used + kRescaleTau) m_new = mt;
    }
    const float off = brow - (m_new == -INFINITY ? 0.0f : m_new);

    // K_{t+2} and V_{t+1} have landed for every wave past this barrier; the
    // scalar loads are taken right after it, where no LDS read is pending (a
    // scalar load in flight would turn the fragment waits of phase B into
    // full drains: scalar loads complete out of order)
    wait_staged();
    sm_next = load_summary(ks_c, tw2);
    kmax_next = kmax_c[tw2];
    if (Q8) kscale_next = kscale_c[tw2];
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::"s"(sm_next.kind), "s"(sm_next.lo), "s"(sm_next.hi), "s"(sm_next.pic), "s"(kmax_next),
                 "s"(kscale_next));
    stage_v(tw2, s2);

    // phase B: O^T += V_t^T P_t^T | row sum of P_t, X_{t+1} = S_{t+1} c +
    // brow - m_new. The ring's last three fetches are the next phase A's
    // first K_{t+2} fragments.
    float ts0 = 0.0f, ts1 = 0.0f;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int j = i + 3;
      if (j < NB) fr[j & 3] = vfrag<VROW, NDB>(vr0, vck, j);
      else if (!Q8) fr[j & 3] = kfrag<KBS>(kn0, kl, j - NB);
      else if (j == NB) kf8[0] = kfrag8<KROWB>(reinterpret_cast<const char*>(KBUF(s2)) + koffb8, k8o, 0);
      const int db = i % NDB, kc = i / NDB;
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr[i & 3], as_bf16x8(pw[kc]), o[db], 0, 0, 0);
      // spread 32 sums and 32 scale-FMAs over the fragments
      constexpr int PER = (32 + NB - 1) / NB;
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int f = i * PER + u;
        if (f < 32) {
          if (f & 1) ts1 += x[f >> 4][f & 15];
          else ts0 += x[f >> 4][f & 15];
          x[f >> 4][f & 15] = fmaf(sn[f >> 4][f & 15], cc, off);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // X_{t+1} belongs to phase B (its FMAs hide under the PV MFMAs): keep it
    // from being sunk past the rescale branch
    keep16(x[0]);
    keep16(x[1]);
    lsum += ts0 + ts1;
    if (wave_any(m_new > m_used)) {
      // lazy rescale after the PV product of tile t (which used the old m);
      // rows whose m stays put (possibly still -inf) keep their sums as they are
      const float alpha = m_new > m_used ? fast_exp2(m_used - m_new) : 1.0f;
      lsum *= alpha;
#pragma unroll
      for (int i = 0; i < NDB; ++i) o[i] *= alpha;
      m_used = m_new;
    }
    tw1 = tw2;
    tw2 = tw3;
    tw3 = TERM ? __builtin_amdgcn_readfirstlane(tv4) : tile_at(t + 4);
  };
  for (int t = 0; t < ntiles; t += NS) {
    step(SlotIndex<0>{}, t);
    if (t + 1 < ntiles) step(SlotIndex<1>{}, t + 1);
    if (t + 2 < ntiles) step(SlotIndex<2>{}, t + 2);
  }
  // no DMA may still target this workgroup's LDS when it exits
  wait_vm<0>();

  // epilogue (a row without any contribution: O 0, LSE -inf)
  const float ltot = xor32_sum(lsum);
  if (!qvalid) return;
  const bool nonempty = ltot > 0.0f;
  const float inv = nonempty ? 1.0f / ltot : 0.0f;
  const float lse = nonempty ? (m_used + __log2f(ltot)) * kLn2 : -INFINITY;
  if (!nonempty) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
  }
  if (PART) {
    float* op = a.opart + ((((int64_t)part * a.B + b) * a.H + h) * a.prows + (qrow - a.prow0)) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f32x4 y;
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = o[db][j * 4 + i] * inv;
        *reinterpret_cast<f32x4*>(op + db * 32 + j * 8 + hh * 4) = y;
      }
    if (hh == 0) a.lsepart[(((int64_t)part * a.B + b) * a.H + h) * a.prows + (qrow - a.prow0)] = lse;
  } else {
    __bf16* op = static_cast<__bf16*>(a.o) + b * a.o_sb + h * a.o_sh + (int64_t)qrow * a.o_sn;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x4 y;
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = (__bf16)(o[db][j * 4 + i] * inv);
        *reinterpret_cast<bf16x4*>(op + db * 32 + j * 8 + hh * 4) = y;
      }
    if (hh == 0) a.lse[((int64_t)b * a.H + h) * N + qrow] = lse;
  }
}

#undef KBUF
#undef VBUF

// ------------------------------------------------------ tile-class counts
// Debug readback of the bias classes the fused / range pass takes: one wave per
// group of 32 query rows (the rows one wave of attn_bf16_kernel holds; lanes
// l and l + 32 hold the same row there, and here). For every key tile of every
// partition it makes the kernel's decision with the same tile_class_lane, and
// counts (row, key tile) pairs per class into counts[b][group][TC_*]: the
// per-element path when some row of the group needs it, else each row's
// constant class. Rows past N are not counted.
__global__ __launch_bounds__(64) void tile_stats_kernel(AttnArgs a, int pass, unsigned* __restrict__ counts) {
  const int g = blockIdx.x, b = blockIdx.y, lane = threadIdx.x & 31;
  const int ngroups = gridDim.x;
  const int row = g * 32 + lane;
  const bool valid = row < a.N;
  const int qr = valid ? row : a.N - 1;
  const float tq = a.tq[(int64_t)b * a.N + qr];
  const bool qbiased = tq == tq;
  const float* gtq = a.gt + ((int64_t)b * a.N + qr) * a.npics;
  unsigned c[TC_COUNT] = {};
  for (int p = 0; p < a.nparts; ++p) {
    const int k0 = a.kr[p], k1 = a.kr[p + 1];
    if (k1 <= k0) continue;
    for (int kt = k0 / kBlockK; kt < (k1 + kBlockK - 1) / kBlockK; ++kt) {
      const KeyTileSummary sm = a.ksum[(int64_t)b * a.nkt + kt];
      const int kbase = kt * kBlockK;
      const bool partial = a.elem_all || kbase < k0 || kbase + kBlockK > k1;
      const float gpic = a.npics > 0 ? gtq[max(sm.pic, 0)] : 0.0f;
      float brow;
      const bool lane_elem = pass == PASS_RANGE ? tile_class_lane<PASS_RANGE>(sm, partial, qbiased, tq, gpic, a, &brow)
                                                : tile_class_lane<PASS_FUSED>(sm, partial, qbiased, tq, gpic, a, &brow);
      int cls;
      if (wave_any(lane_elem)) cls = TC_ELEM;
      else if ((sm.kind & KT_CLASS) == KT_PICTURE) cls = TC_PICTURE;
      else if ((sm.kind & KT_CLASS) == KT_GUIDE && qbiased) cls = brow != 0.0f ? TC_SATURATED : TC_WINDOW;
      else cls = TC_PLAIN;
      if (valid) ++c[cls];
    }
  }
  // sum over the group's 32 rows (lanes 32..63 repeat lanes 0..31)
#pragma unroll
  for (int i = 0; i < TC_COUNT; ++i) {
    unsigned x = c[i];
    for (int off = 16; off >= 1; off >>= 1) x += __shfl_xor(x, off, 32);
    if (threadIdx.x == 0) counts[((int64_t)b * ngroups + g) * TC_COUNT + i] = x;
  }
}

hipError_t launch_tile_stats(const AttnArgs& a, int pass, unsigned* counts, hipStream_t s) {
  dim3 grid(tile_stats_groups(a.N), a.B);
  hipLaunchKernelGGL(tile_stats_kernel, grid, dim3(64), 0, s, a, pass, counts);
  return hipGetLastError();
}

// Workgroup shape of the bf16 kernel: kWaves waves of 32 query rows.
constexpr int kWaves = 8;

int attn_bf16_block_q(int) { return kWaves * 32; }

int attn_bf16_grid(const AttnArgs& a) { return a.nqb * a.B * a.H; }

template <int D>
void launch_attn_bf16_d(const AttnArgs& a, int pass, int variant, dim3 grid, dim3 block, hipStream_t s) {
  switch (pass) {
    case PASS_FUSED:
      if (variant == ATTN_QK8)
        hipLaunchKernelGGL((attn_bf16_kernel<D, kWaves, PASS_FUSED, true, false>), grid, block, 0, s, a);
      else if (variant == ATTN_DENSE_BIAS)
        hipLaunchKernelGGL((attn_bf16_kernel<D, kWaves, PASS_FUSED, false, true>), grid, block, 0, s, a);
      else
        hipLaunchKernelGGL((attn_bf16_kernel<D, kWaves, PASS_FUSED, false, false>), grid, block, 0, s, a);
      break;
    case PASS_RANGE:
      if (variant == ATTN_QK8)
        hipLaunchKernelGGL((attn_bf16_kernel<D, kWaves, PASS_RANGE, true, false>), grid, block, 0, s, a);
      else
        hipLaunchKernelGGL((attn_bf16_kernel<D, kWaves, PASS_RANGE, false, false>), grid, block, 0, s, a);
      break;
    case PASS_TERM_A:
      hipLaunchKernelGGL((attn_bf16_kernel<D, kWaves, PASS_TERM_A, false, false>), grid, block, 0, s, a);
      break;
    case PASS_TERM_B:
      hipLaunchKernelGGL((attn_bf16_kernel<D, kWaves, PASS_TERM_B, false, false>), grid, block, 0, s, a);
      break;
    default:
      hipLaunchKernelGGL((attn_bf16_kernel<D, kWaves, PASS_TERM_C, false, false>), grid, block, 0, s, a);
      break;
  }
}

hipError_t launch_attn_bf16(const AttnArgs& a, int D, int pass, int variant, hipStream_t s) {
  // the dense-bias baseline exists for the one-pass form only, 8-bit Q.K for
  // it and the range pass of a fused call's tail (the host rejects the rest)
  if (variant == ATTN_DENSE_BIAS && pass != PASS_FUSED) return hipErrorInvalidValue;
  if (variant == ATTN_QK8 && pass != PASS_FUSED && pass != PASS_RANGE) return hipErrorInvalidValue;
  dim3 grid(attn_bf16_grid(a), pass == PASS_RANGE ? a.nparts : 1);
  dim3 block(kWaves * 64);
  if (D == 128) launch_attn_bf16_d<128>(a, pass, variant, grid, block, s);
  else launch_attn_bf16_d<64>(a, pass, variant, grid, block, s);
  return hipGetLastError();
}

// Dense-bias baseline: the bias of every (query, key) pair of batch element
// blockIdx.z in log2 units, as the per-element path computes it (temporal
// penalty of a biased target row against a biased guide key, plus the row's
// summed log2 gain of a bound picture key), written as fp32 rows of npad keys;
// keys at or past N get -inf. Four keys per thread.
__global__ __launch_bounds__(256) void dense_bias_kernel(AttnArgs a, float* __restrict__ out) {
  const int q = blockIdx.x, b = blockIdx.z;
  const int k = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (k >= a.npad) return;
  const int64_t qi = (int64_t)b * a.N + q;
  const float tq = a.tq[qi];
  const float* gq = a.gt + qi * a.npics;
  f32x4 r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int kk = k + e;
    float x = -INFINITY;
    if (kk < a.N) {
      const float tk = a.tk[(int64_t)b * a.npad + kk];
      const float dd = fmaxf(fmaf(fabsf(tq - tk), a.sigma, -a.w), 0.0f);   // NaN time -> 0
      x = -fminf(dd * dd, a.cap2);
      const int kp = a.kp[(int64_t)b * a.npad + kk];
      if (kp >= 0) x += gq[kp];
    }
    r[e] = x;
  }
  *reinterpret_cast<f32x4*>(out + qi * a.npad + k) = r;
}

hipError_t launch_dense_bias(const AttnArgs& a, float* out, hipStream_t s) {
  dim3 grid(a.N, (a.npad + 1023) / 1024, a.B);
  hipLaunchKernelGGL(dense_bias_kernel, grid, dim3(256), 0, s, a, out);
  return hipGetLastError();
}

// ----------------------------------------------------------------- fp32 path
// 64 query rows per workgroup, four lanes per row, each holding D/4 dims of q
// and of the output. Key tiles of 64 keys (K and V rows, key times, picture
// ids) are staged in LDS by the whole workgroup; each lane forms its row's
// logits 16 keys at a time (partial dot products over its dims, summed across
// the row's four lanes), rescales once per 16 keys to the new row max and adds
// their weighted V rows to its output dims.
constexpr int kF32Queries = 64;
constexpr int kF32Keys = 64;
constexpr int kF32Chunk = 16;

template <int D, int PASS>
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a) {
  constexpr int DL = D / 4;
  constexpr int KP = D + 4;   // LDS pitch of a staged row (floats): the four lanes' slices hit different banks
  constexpr bool PART = PASS != PASS_FUSED;
  constexpr bool TERM = PASS >= PASS_TERM_A;
  __shared__ __attribute__((aligned(16))) float ks[kF32Keys * KP];
  __shared__ __attribute__((aligned(16))) float vs[kF32Keys * KP];
  __shared__ float tks[kF32Keys];
  __shared__ int kps[kF32Keys];   // picture id (>= 0), -1 for other keys, -2 for keys outside this pass's range
  const int part = PASS == PASS_RANGE ? blockIdx.z : TERM ? PASS - PASS_TERM_A : 0;
  const int bh = blockIdx.y, b = bh / a.H, h = bh % a.H;
  const int N = a.N;
  const int tid = threadIdx.x, sub = tid & 3;
  const int qrow = a.qr0 + blockIdx.x * kF32Queries + (tid >> 2);   // rows [qr0, qr1) of this launch
  const bool qvalid = qrow < a.qr1;
  const int qr = qvalid ? qrow : a.qr1 - 1;
  const float* qp = static_cast<const float*>(a.q) + b * a.q_sb + h * a.q_sh + (int64_t)qr * a.q_sn + sub * DL;
  const float* kg = static_cast<const float*>(a.k) + b * a.k_sb + h * a.k_sh;
  const float* vg = static_cast<const float*>(a.v) + b * a.v_sb + h * a.v_sh;
  float qv[DL], ov[DL];
#pragma unroll
  for (int i = 0; i < DL; i += 4) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(qp + i);
    qv[i] = x[0]; qv[i + 1] = x[1]; qv[i + 2] = x[2]; qv[i + 3] = x[3];
    ov[i] = ov[i + 1] = ov[i + 2] = ov[i + 3] = 0.0f;
  }
  const float tq = a.tq[(int64_t)b * N + qr];
  const float* tkb = a.tk + (int64_t)b * a.npad;
  const int* kpb = a.kp + (int64_t)b * a.npad;
  const float* gtq = a.gt + ((int64_t)b * N + qr) * a.npics;
  const int k0 = TERM ? 0 : a.kr[part], k1 = TERM ? N : a.kr[part + 1];
  const bool qb = tq == tq;
  float m = -INFINITY, l = 0.0f;
  for (int kbase = k0 / kF32Keys * kF32Keys; kbase < k1; kbase += kF32Keys) {
    __syncthreads();   // every lane is done with the previous tile
    // stage the tile: rows of D floats as 16-byte chunks, zeros past [k0, k1)
#pragma unroll
    for (int it = 0; it < kF32Keys * D / 4 / 256; ++it) {
      const int c = tid + it * 256;
      const int r = c / (D / 4), col = (c % (D / 4)) * 4, key = kbase + r;
      f32x4 kx = {}, vx = {};
      if (key >= k0 && key < k1) {
        kx = *reinterpret_cast<const f32x4*>(kg + (int64_t)key * a.k_sn + col);
        vx = *reinterpret_cast<const f32x4*>(vg + (int64_t)key * a.v_sn + col);
      }
      *reinterpret_cast<f32x4*>(ks + r * KP + col) = kx;
      *reinterpret_cast<f32x4*>(vs + r * KP + col) = vx;
    }
    if (tid < kF32Keys) {
      const int key = kbase + tid;
      const bool in = key >= k0 && key < k1;
      tks[tid] = in ? tkb[key] : 0.0f;
      kps[tid] = in ? kpb[key] : -2;
    }
    __syncthreads();
    // chunks of kF32Chunk keys: the row's logits (log2 units; -inf: not a key
    // of this pass), one rescale to the chunk's new row max (a row with no
    // finite logit yet keeps m = -inf and exponent reference 0, so its
    // weights stay 0), then the chunk's weighted V rows
#pragma unroll 1
    for (int j0 = 0; j0 < kF32Keys; j0 += kF32Chunk) {
      float x[kF32Chunk];
      float mt = -INFINITY;
#pragma unroll
      for (int jj = 0; jj < kF32Chunk; ++jj) {
        const int j = j0 + jj;
        const float* kr = ks + j * KP + sub * DL;
        float sdot = 0.0f;
#pragma unroll
        for (int i = 0; i < DL; i += 4) {
          const f32x4 kx = *reinterpret_cast<const f32x4*>(kr + i);
          sdot = fmaf(qv[i], kx[0], sdot);
          sdot = fmaf(qv[i + 1], kx[1], sdot);
          sdot = fmaf(qv[i + 2], kx[2], sdot);
          sdot = fmaf(qv[i + 3], kx[3], sdot);
        }
        sdot = quad_sum(sdot);   // the row's four lanes
        const float tk = tks[j];
        const int pk = kps[j];
        const float dd = fmaxf(fmaf(fabsf(tq - tk), a.sigma, -a.w), 0.0f);
        const float pen = fminf(dd * dd, a.cap2);
        const float gain = pk >= 0 ? gtq[pk] : 0.0f;
        const bool isg = tk == tk;   // a biased guide key
        float xj;
        if (PASS == PASS_TERM_A) xj = isg ? -INFINITY : fmaf(sdot, a.c, gain);
        else if (PASS == PASS_TERM_B) xj = isg ? fmaf(sdot, a.c, qb ? -a.cap2 : 0.0f) : -INFINITY;
        else if (PASS == PASS_TERM_C)
          xj = isg && qb ? fmaf(sdot, a.c, __log2f(1.0f - exp2f(pen - a.cap2)) - pen) : -INFINITY;
        else xj = fmaf(sdot, a.c, gain - pen);
        if (pk == -2) xj = -INFINITY;
        x[jj] = xj;
        mt = fmaxf(mt, xj);
      }
      const float mn = fmaxf(m, mt);
      const float mref = mn == -INFINITY ? 0.0f : mn;
      const float alpha = exp2f(m - mref);
      float ts = 0.0f;
#pragma unroll
      for (int i = 0; i < DL; ++i) ov[i] *= alpha;
#pragma unroll
      for (int jj = 0; jj < kF32Chunk; ++jj) {
        const float p = exp2f(x[jj] - mref);
        ts += p;
        const float* vr = vs + (j0 + jj) * KP + sub * DL;
#pragma unroll
        for (int i = 0; i < DL; i += 4) {
          const f32x4 vx = *reinterpret_cast<const f32x4*>(vr + i);
          ov[i] = fmaf(p, vx[0], ov[i]);
          ov[i + 1] = fmaf(p, vx[1], ov[i + 1]);
          ov[i + 2] = fmaf(p, vx[2], ov[i + 2]);
          ov[i + 3] = fmaf(p, vx[3], ov[i + 3]);
        }
      }
      l = fmaf(l, alpha, ts);
      m = mn;
    }
  }
  if (!qvalid) return;
  const bool empty = !(l > 0.0f);
  const float inv = empty ? 0.0f : 1.0f / l;
  const float lse = empty ? -INFINITY : (m + log2f(l)) * kLn2;
  float* op;
  if (PART) op = a.opart + ((((int64_t)part * a.B + b) * a.H + h) * a.prows + (qrow - a.prow0)) * D + sub * DL;
  else op = static_cast<float*>(a.o) + b * a.o_sb + h * a.o_sh + (int64_t)qrow * a.o_sn + sub * DL;
#pragma unroll
  for (int i = 0; i < DL; i += 4)
    *reinterpret_cast<f32x4*>(op + i) = f32x4{ov[i] * inv, ov[i + 1] * inv, ov[i + 2] * inv, ov[i + 3] * inv};
  if (sub == 0) {
    if (PART) a.lsepart[(((int64_t)part * a.B + b) * a.H + h) * a.prows + (qrow - a.prow0)] = lse;
    else a.lse[((int64_t)b * a.H + h) * N + qrow] = lse;
  }
}

int attn_f32_block_q(int) { return kF32Queries; }

template <int D>
void launch_attn_f32_d(const AttnArgs& a, int pass, dim3 grid, dim3 block, hipStream_t s) {
  switch (pass) {
    case PASS_FUSED: hipLaunchKernelGGL((attn_f32_kernel<D, PASS_FUSED>), grid, block, 0, s, a); break;
    case PASS_RANGE: hipLaunchKernelGGL((attn_f32_kernel<D, PASS_RANGE>), grid, block, 0, s, a); break;
    case PASS_TERM_A: hipLaunchKernelGGL((attn_f32_kernel<D, PASS_TERM_A>), grid, block, 0, s, a); break;
    case PASS_TERM_B: hipLaunchKernelGGL((attn_f32_kernel<D, PASS_TERM_B>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((attn_f32_kernel<D, PASS_TERM_C>), grid, block, 0, s, a); break;
  }
}

hipError_t launch_attn_f32(const AttnArgs& a, int D, int pass, hipStream_t s) {
  dim3 grid((a.qr1 - a.qr0 + kF32Queries - 1) / kF32Queries, a.B * a.H, pass == PASS_RANGE ? a.nparts : 1);
  dim3 block(256);
  if (D == 128) launch_attn_f32_d<128>(a, pass, grid, block, s);
  else launch_attn_f32_d<64>(a, pass, grid, block, s);
  return hipGetLastError();
}

// --------------------------------------------------------------- LSE merge
// One thread per (row, 8 consecutive dims): LSE = M + ln sum_p e^(LSE_p - M),
// O = sum_p e^(LSE_p - LSE) O_p (a row whose partitions are all empty gets O
// 0 and LSE -inf). NP > 0: exactly NP partitions, unrolled so that every load
// of the row is in flight at once; NP == 0: a.nparts, looped.
template <bool BF16_OUT, int NP>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int dq = a.D / 8;
  const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t rows = (int64_t)a.B * a.H * a.rows;
  if (gid >= rows * dq) return;
  const int d8 = (int)(gid % dq);
  const int64_t row = gid / dq;                   // (b*H + h)*rows + n - row0: the partials' row
  const int n = a.row0 + (int)(row % a.rows);
  const int64_t bh = row / a.rows;
  const int b = (int)(bh / a.H), h = (int)(bh % a.H);
  const int np = NP > 0 ? NP : a.nparts;
  f32x4 acc0 = f32x4{}, acc1 = f32x4{};
  float lse = -INFINITY;
  if constexpr (NP > 0) {
    float l[NP];
    f32x4 x0[NP], x1[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      l[p] = a.lsepart[(int64_t)p * rows + row];
      const float* op = a.opart + ((int64_t)p * rows + row) * a.D + d8 * 8;
      x0[p] = *reinterpret_cast<const f32x4*>(op);
      x1[p] = *reinterpret_cast<const f32x4*>(op + 4);
    }
    float mx = l[0];
#pragma unroll
    for (int p = 1; p < NP; ++p) mx = fmaxf(mx, l[p]);
    if (mx != -INFINITY) {
      float ssum = 0.0f;
#pragma unroll
      for (int p = 0; p < NP; ++p) ssum += expf(l[p] - mx);
      lse = mx + logf(ssum);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const float w = expf(l[p] - lse);
        acc0 += w * x0[p];
        acc1 += w * x1[p];
      }
    }
  } else {
    float mx = -INFINITY;
    for (int p = 0; p < np; ++p) mx = fmaxf(mx, a.lsepart[(int64_t)p * rows + row]);
    if (mx != -INFINITY) {
      float ssum = 0.0f;
      for (int p = 0; p < np; ++p) ssum += expf(a.lsepart[(int64_t)p * rows + row] - mx);
      lse = mx + logf(ssum);
      for (int p = 0; p < np; ++p) {
        const float w = expf(a.lsepart[(int64_t)p * rows + row] - lse);
        const float* op = a.opart + ((int64_t)p * rows + row) * a.D + d8 * 8;
        acc0 += w * *reinterpret_cast<const f32x4*>(op);
        acc1 += w * *reinterpret_cast<const f32x4*>(op + 4);
      }
    }
  }
  const int64_t oo = b * a.o_sb + h * a.o_sh + (int64_t)n * a.o_sn + d8 * 8;
  if (BF16_OUT) {
    bf16x8 y;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      y[i] = (__bf16)acc0[i];
      y[i + 4] = (__bf16)acc1[i];
    }
    *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(a.o) + oo) = y;
  } else {
    float* o = static_cast<float*>(a.o) + oo;
    *reinterpret_cast<f32x4*>(o) = acc0;
    *reinterpret_cast<f32x4*>(o + 4) = acc1;
  }
  if (d8 == 0) a.lse[bh * a.N + n] = lse;
}

template <bool BF16_OUT>
void launch_merge_np(const MergeArgs& a, dim3 grid, hipStream_t s) {
  if (a.nparts == 2) hipLaunchKernelGGL((merge_kernel<BF16_OUT, 2>), grid, dim3(256), 0, s, a);
  else if (a.nparts == 3) hipLaunchKernelGGL((merge_kernel<BF16_OUT, 3>), grid, dim3(256), 0, s, a);
  else if (a.nparts == 4) hipLaunchKernelGGL((merge_kernel<BF16_OUT, 4>), grid, dim3(256), 0, s, a);
  else hipLaunchKernelGGL((merge_kernel<BF16_OUT, 0>), grid, dim3(256), 0, s, a);
}

hipError_t launch_merge(const MergeArgs& a, bool bf16_out, hipStream_t s) {
  const int64_t total = (int64_t)a.B * a.H * a.rows * (a.D / 8);
  dim3 grid((unsigned)((total + 255) / 256));
  if (bf16_out) launch_merge_np<true>(a, grid, s);
  else launch_merge_np<false>(a, grid, s);
  return hipGetLastError();
}

}  // namespace tara
