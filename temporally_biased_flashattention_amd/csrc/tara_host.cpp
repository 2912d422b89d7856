// Host side of the TARA attention C ABI (include/tara.h): argument checks,
// derived constants, workspace carving and kernel dispatch. No device memory
// is allocated here; every launch goes to the caller's stream.
#include "tara.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <numeric>
#include <string>
#include <utility>
#include <vector>

#include "tara_internal.h"

namespace {

thread_local std::string g_err;
thread_local tara_run_info_t g_info;
thread_local bool g_info_valid = false;

int fail(int status, const std::string& msg) {
  g_err = msg;
  return status;
}

bool env_flag(const char* name) {
  const char* v = std::getenv(name);
  return v && v[0] && std::strcmp(v, "0") != 0;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct WsLayout {
  size_t tq, tk, kp, gt, ksum, vt, kmax, k8, ks, dbias, opart, lsepart, tstats, total;
};

int npad_of(int N) { return (N + tara::kBlockK - 1) / tara::kBlockK * tara::kBlockK; }

int num_parts(const tara_params_t* p) {
  return p->mode == TARA_MODE_PARTITIONED ? p->num_partitions : p->mode == TARA_MODE_THREE_TERM ? 3 : 1;
}

// Modes whose attention passes write per-partition (O_p, LSE_p) for a merge.
bool has_partials(const tara_params_t* p) {
  return p->mode == TARA_MODE_PARTITIONED || p->mode == TARA_MODE_THREE_TERM;
}

// Fused bf16 calls (8-bit Q.K too) whose workgroups would leave the last round of
// compute units partly filled: the first m query blocks of every (batch, head)
// run as the fused pass and fill whole rounds; the remaining ones run as the
// range pass over `parts` key ranges (parts times as many workgroups, each over
// 1/parts of the keys) followed by the exact LSE merge of those rows. Planned
// for kTargetCUs compute units (MI355X) from the call shape alone, so that
// tara_workspace_bytes and the call agree; the results are the same up to
// rounding either way.
constexpr int kTargetCUs = 256;
constexpr int kMaxTailParts = 16;
struct TailSplit {
  int m = 0;       // query blocks per (batch, head) in the fused pass
  int parts = 0;   // key ranges of the rest (0: no split)
  int row0 = 0;    // first row of the rest
};
TailSplit tail_split(tara_dtype_t dtype, int B, int H, int N, int D, const tara_params_t* p) {
  TailSplit t;
  if (dtype != TARA_BF16 || p->mode != TARA_MODE_FUSED || B <= 0 || H <= 0 || N <= 0) return t;
  const int64_t bq = tara::attn_bf16_block_q(D), bh = (int64_t)B * H, nqb = (N + bq - 1) / bq;
  const int64_t total = bh * nqb;
  if (total <= kTargetCUs) return t;   // within one round: left as it is
  // m: the most query blocks per (batch, head) whose workgroups fill whole rounds
  const int64_t g = kTargetCUs / std::gcd(bh, (int64_t)kTargetCUs);
  const int64_t m = nqb / g * g;
  if (m == 0 || m == nqb) return t;
  // rounds of one full-length workgroup per compute unit: ceil(total / CUs)
  // unsplit; m's rounds plus the range pass's (its workgroups 1/parts as long)
  const double unsplit = std::ceil((double)total / kTargetCUs);
  const double main_rounds = (double)(bh * m / kTargetCUs);
  const int64_t rest = bh * (nqb - m);
  // at most two rounds of query blocks are split off, into at most four
  // rounds of range-pass workgroups: the partial outputs stay small (at most
  // 1,024 query blocks of fp32 O and LSE)
  if (rest > 2 * kTargetCUs) return t;
  double best = unsplit;
  int best_parts = 0;
  for (int pp = 2; pp <= kMaxTailParts && rest * pp <= 4 * kTargetCUs; ++pp) {
    const double r = main_rounds + std::ceil((double)(rest * pp) / kTargetCUs) / pp;
    if (r < best - 1e-9) {
      best = r;
      best_parts = pp;
    }
  }
  if (best_parts == 0 || unsplit - best < 0.05) return t;   // too little to gain against the extra launches
  t.m = (int)m;
  t.parts = best_parts;
  t.row0 = (int)(m * bq);
  return t;
}

// 8-bit Q.K: the bf16 path in fused mode only
bool uses_qk8(tara_dtype_t dtype, const tara_params_t* p) { return p->qk8 && dtype == TARA_BF16; }
bool qk8_supported(tara_dtype_t dtype, const tara_params_t* p) {
  return !p->qk8 || (dtype == TARA_BF16 && p->mode == TARA_MODE_FUSED);
}

int num_bindings(const tara_params_t* p) { return p->num_bindings < 1 ? 1 : p->num_bindings; }

// Pictures of the gain table (0 without binding).
int table_pictures(const tara_params_t* p) { return p->binding_enabled ? p->num_pictures : 0; }

// Workspace regions, each 256-byte aligned: per-token encodings (with
// binding, the per-query gain table), key-tile summaries, V^T (bf16 path),
// the FP8 copy of K and its tile scales (8-bit Q.K), and per-partition O/LSE
// (every mode but fused; in fused mode those of the rows a tail split hands
// to the range pass).
WsLayout ws_layout_for(tara_dtype_t dtype, int B, int H, int N, int D, const tara_params_t* p, const TailSplit& t) {
  WsLayout L{};
  const size_t npad = (size_t)npad_of(N), nkt = npad / tara::kBlockK;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  L.tq = take((size_t)B * N * 4);
  L.tk = take((size_t)B * npad * 4);
  L.kp = take((size_t)B * npad * 4);
  L.gt = take((size_t)B * N * table_pictures(p) * 4);
  L.ksum = take((size_t)B * nkt * sizeof(tara::KeyTileSummary));
  // tile-class counts of the debug readback (bf16 FUSED / PARTITIONED)
  L.tstats = take((size_t)B * tara::tile_stats_groups(N) * tara::TC_COUNT * 4);
  L.vt = dtype == TARA_BF16 ? take((size_t)B * H * D * npad * 2) : 0;
  L.kmax = dtype == TARA_BF16 ? take((size_t)B * H * nkt * 4) : 0;
  if (uses_qk8(dtype, p)) {
    L.k8 = take((size_t)B * H * npad * D);
    L.ks = take((size_t)B * H * nkt * 4);
  }
  if (p->mode == TARA_MODE_DENSE_BIAS) L.dbias = take((size_t)B * N * npad * 4);
  if (has_partials(p)) {
    const size_t parts = (size_t)num_parts(p);
    L.opart = take(parts * B * H * N * D * 4);
    L.lsepart = take(parts * B * H * N * 4);
  } else {
    if (t.parts) {   // the partial outputs of the split-off rows only
      const size_t rows = (size_t)(N - t.row0);
      L.opart = take((size_t)t.parts * B * H * rows * D * 4);
      L.lsepart = take((size_t)t.parts * B * H * rows * 4);
    }
  }
  L.total = off;
  return L;
}

bool finite(float x) { return std::isfinite(x); }

int check_params(const tara_params_t* p, int N) {
  if (!finite(p->window) || !finite(p->falloff) || !finite(p->strength) || !finite(p->cap))
    return fail(TARA_ERR_BAD_PARAM, "window, falloff, strength and cap must be finite");
  if (p->window < 0.0f) return fail(TARA_ERR_BAD_PARAM, "window must be >= 0");
  if (!(p->falloff > 0.0f)) return fail(TARA_ERR_BAD_PARAM, "falloff must be > 0");
  if (p->strength < 0.0f) return fail(TARA_ERR_BAD_PARAM, "strength must be >= 0");
  if (p->cap < 0.0f) return fail(TARA_ERR_BAD_PARAM, "cap must be >= 0");
  if (!finite(p->softmax_scale) || p->softmax_scale < 0.0f)
    return fail(TARA_ERR_BAD_PARAM, "softmax_scale must be finite and >= 0 (0 = 1/sqrt(D))");
  if (p->binding_enabled) {
    if (p->num_pictures < 0 || p->num_pictures > TARA_MAX_PICTURES)
      return fail(TARA_ERR_BAD_PARAM, "num_pictures must be in [0, 16]");
    if (p->num_bindings < 0 || p->num_bindings > TARA_MAX_BINDINGS)
      return fail(TARA_ERR_BAD_PARAM, "num_bindings must be in [0, 4] (0 is read as 1)");
    for (int j = 0; j < num_bindings(p); ++j)
      for (int i = 0; i < p->num_pictures; ++i)
        if (!finite(p->picture_gain[j][i]) || !(p->picture_gain[j][i] > 0.0f))
          return fail(TARA_ERR_BAD_PARAM, "picture gains must be finite and > 0 (the rule adds m*ln(gain))");
  }
  if (p->mode < TARA_MODE_FUSED || p->mode > TARA_MODE_FRAME_LOOP)
    return fail(TARA_ERR_BAD_PARAM, "mode must be one of tara_mode_t");
  if (p->mode == TARA_MODE_PARTITIONED || p->mode == TARA_MODE_FRAME_LOOP) {
    if (p->mode == TARA_MODE_PARTITIONED && (p->num_partitions < 1 || p->num_partitions > TARA_MAX_PARTITIONS))
      return fail(TARA_ERR_BAD_PARAM, "num_partitions must be in [1, 64]");
    if (p->mode == TARA_MODE_FRAME_LOOP && (p->num_partitions < 1 || p->num_partitions > std::max(N, 1)))
      return fail(TARA_ERR_BAD_PARAM, "FRAME_LOOP needs 1 <= num_partitions <= max(N, 1)");
    if (p->partition_bounds) {
      const int32_t* pb = p->partition_bounds;
      if (pb[0] != 0 || pb[p->num_partitions] != N)
        return fail(TARA_ERR_BAD_PARAM, "partition_bounds must start at 0 and end at N");
      for (int i = 0; i < p->num_partitions; ++i)
        if (pb[i + 1] < pb[i]) return fail(TARA_ERR_BAD_PARAM, "partition_bounds must be non-decreasing");
    }
  }
  return TARA_OK;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15) == 0; }

int check_strides(const char* name, const void* base, const int64_t* s, int esize) {
  if (!s) return fail(TARA_ERR_NULL_POINTER, std::string(name) + " strides are NULL");
  if (!aligned16(base)) return fail(TARA_ERR_BAD_STRIDE, std::string(name) + " base is not 16-byte aligned");
  const int64_t q = 16 / esize;
  for (int i = 0; i < 3; ++i)
    if (s[i] < 0 || s[i] % q != 0)
      return fail(TARA_ERR_BAD_STRIDE, std::string(name) + " strides must be >= 0 and multiples of " +
                                           std::to_string(q) + " elements");
  return TARA_OK;
}

// Optional synchronous metadata check (TARA_VALIDATE=1).
int validate_metadata(int B, int N, const uint8_t* seg, const float* time, const int16_t* pic,
                      const float* mask, const tara_params_t* p, hipStream_t stream) {
  const size_t n = (size_t)B * N;
  std::vector<uint8_t> hs(n);
  std::vector<float> ht(n), hm;
  std::vector<int16_t> hp;
  if (hipStreamSynchronize(stream) != hipSuccess ||
      hipMemcpy(hs.data(), seg, n, hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(ht.data(), time, n * 4, hipMemcpyDeviceToHost) != hipSuccess)
    return fail(TARA_ERR_HIP, "TARA_VALIDATE: copying metadata to the host failed");
  const bool bind = p->binding_enabled != 0;
  if (bind && pic) {
    hp.resize(n);
    if (hipMemcpy(hp.data(), pic, n * 2, hipMemcpyDeviceToHost) != hipSuccess)
      return fail(TARA_ERR_HIP, "TARA_VALIDATE: copying picture ids failed");
  }
  const int nb = num_bindings(p);
  if (bind && mask) {
    hm.resize(n * nb);
    if (hipMemcpy(hm.data(), mask, n * nb * 4, hipMemcpyDeviceToHost) != hipSuccess)
      return fail(TARA_ERR_HIP, "TARA_VALIDATE: copying the mask failed");
  }
  for (size_t i = 0; i < n; ++i) {
    if (hs[i] > 3) return fail(TARA_ERR_BAD_METADATA, "seg_type[" + std::to_string(i) + "] > 3");
    if ((hs[i] == TARA_SEG_TARGET || hs[i] == TARA_SEG_GUIDE) && !std::isfinite(ht[i]))
      return fail(TARA_ERR_BAD_METADATA, "token_time[" + std::to_string(i) + "] of a video token is not finite");
    if (bind && hs[i] == TARA_SEG_PICTURE && !hp.empty() && (hp[i] < 0 || hp[i] >= p->num_pictures))
      return fail(TARA_ERR_BAD_METADATA, "picture_id[" + std::to_string(i) + "] outside [0, num_pictures)");
    if (bind && hs[i] == TARA_SEG_TARGET && !hm.empty())
      for (int j = 0; j < nb; ++j)
        if (!std::isfinite(hm[(size_t)j * n + i]))
          return fail(TARA_ERR_BAD_METADATA, "mask_weight[" + std::to_string(j) + "][" + std::to_string(i) +
                                                 "] is not finite");
  }
  return TARA_OK;
}

// Event timing of the attention kernel.
std::mutex g_tmu;
bool g_timing = false;
std::vector<std::pair<hipEvent_t, hipEvent_t>> g_events;

}  // namespace

namespace tara {

int set_error(int status, const std::string& msg) { return fail(status, msg); }

void set_last_info(const tara_run_info_t& info) {
  g_info = info;
  g_info_valid = true;
}

void set_empty_info(const Call& c) {
  tara_run_info_t info{};
  info.mode = c.p->mode;
  info.dtype = (int)c.dtype;
  info.num_partitions = num_parts(c.p);
  info.block_k = kBlockK;
  set_last_info(info);
}

int make_call(Call& c, const void* q, const void* k, const void* v, void* o, float* lse, int dtype_, int B,
              int H, int N, int D, const int64_t q_str[3], const int64_t k_str[3], const int64_t v_str[3],
              const int64_t o_str[3], const uint8_t* seg_type, const float* token_time, const int16_t* picture_id,
              const float* mask_weight, const tara_params_t* p) {
  if (!p) return fail(TARA_ERR_NULL_POINTER, "params are NULL");
  if (dtype_ != TARA_BF16 && dtype_ != TARA_FP32) return fail(TARA_ERR_UNSUPPORTED_DTYPE, "dtype must be TARA_BF16 or TARA_FP32");
  const tara_dtype_t dtype = (tara_dtype_t)dtype_;
  if (D != 64 && D != 128) return fail(TARA_ERR_UNSUPPORTED_HEAD_DIM, "head dim must be 64 or 128");
  if (B < 0 || H < 0 || N < 0) return fail(TARA_ERR_BAD_SHAPE, "B, H and N must be >= 0");
  if ((int64_t)B * H > 65535) return fail(TARA_ERR_BAD_SHAPE, "B * H must be <= 65535");
  if (N > (1 << 30)) return fail(TARA_ERR_BAD_SHAPE, "N must be <= 2^30");
  if (p->mode == TARA_MODE_THREE_TERM && npad_of(N) / kBlockK > kMaxListTiles)
    return fail(TARA_ERR_BAD_SHAPE, "three-term mode supports N <= 2^20 (its key-tile lists live in LDS)");
  if (int st = check_params(p, N)) return st;
  if (!qk8_supported(dtype, p)) return fail(TARA_ERR_BAD_PARAM, "qk8 requires TARA_BF16 and TARA_MODE_FUSED");
  if (p->mode == TARA_MODE_DENSE_BIAS && dtype != TARA_BF16)
    return fail(TARA_ERR_BAD_PARAM, "TARA_MODE_DENSE_BIAS requires TARA_BF16");
  c.p = p;
  c.dtype = dtype;
  c.B = B;
  c.H = H;
  c.N = N;
  c.D = D;
  const TailSplit t = tail_split(dtype, B, H, N, D, p);
  c.tail_m = t.m;
  c.tail_parts = t.parts;
  c.tail_row0 = t.row0;
  if (B == 0 || H == 0 || N == 0) return TARA_OK;
  if (!q || !k || !v || !o || !lse) return fail(TARA_ERR_NULL_POINTER, "q, k, v, o and lse must be non-NULL");
  if (!seg_type || !token_time) return fail(TARA_ERR_NULL_POINTER, "seg_type and token_time must be non-NULL");
  const int esize = dtype == TARA_BF16 ? 2 : 4;
  if (int st = check_strides("q", q, q_str, esize)) return st;
  if (int st = check_strides("k", k, k_str, esize)) return st;
  if (int st = check_strides("v", v, v_str, esize)) return st;
  if (int st = check_strides("o", o, o_str, esize)) return st;
  if ((reinterpret_cast<uintptr_t>(lse) & 3) != 0) return fail(TARA_ERR_BAD_STRIDE, "lse is not 4-byte aligned");
  // the bf16 kernel stages key tiles with 32-bit byte offsets from one head's
  // K rows and from its rows of the key-contiguous V copy: N (padded to whole
  // tiles) rows of K at its row stride, and D rows of that copy, must each
  // span less than 2^31 bytes
  if (dtype == TARA_BF16 && ((int64_t)k_str[2] * 2 * npad_of(N) >= (int64_t(1) << 31) ||
                             (int64_t)D * npad_of(N) * 2 >= (int64_t(1) << 31)))
    return fail(TARA_ERR_BAD_STRIDE, "K row stride x N or D x N too large for the bf16 kernel's 32-bit tile offsets");
  bool binding_active = false;
  if (p->binding_enabled)
    for (int j = 0; j < num_bindings(p); ++j)
      for (int i = 0; i < p->num_pictures; ++i) binding_active |= p->picture_gain[j][i] != 1.0f;
  if (binding_active && !picture_id)
    return fail(TARA_ERR_NULL_POINTER, "picture_id must be non-NULL when binding is active");
  c.q = q;
  c.k = k;
  c.v = v;
  c.o = o;
  c.lse = lse;
  for (int i = 0; i < 3; ++i) {
    c.qs[i] = q_str[i];
    c.ks[i] = k_str[i];
    c.vs[i] = v_str[i];
    c.os[i] = o_str[i];
  }
  c.seg = seg_type;
  c.time = token_time;
  c.pic = picture_id;
  c.mask = mask_weight;
  c.mask_plane = (int64_t)B * N;
  return TARA_OK;
}

TailSplit call_tail(const Call& c) {
  TailSplit t;
  t.m = c.tail_m;
  t.parts = c.tail_parts;
  t.row0 = c.tail_row0;
  return t;
}

size_t call_workspace(const Call& c) { return ws_layout_for(c.dtype, c.B, c.H, c.N, c.D, c.p, call_tail(c)).total; }

Call sub_call(const Call& c, int b, int h0, int hc) {
  Call s = c;
  const int esize = c.dtype == TARA_BF16 ? 2 : 4;
  auto at = [&](const void* base, const int64_t* st) {
    return static_cast<const void*>(static_cast<const char*>(base) + (b * st[0] + h0 * st[1]) * esize);
  };
  s.q = at(c.q, c.qs);
  s.k = at(c.k, c.ks);
  s.v = at(c.v, c.vs);
  s.o = const_cast<void*>(at(c.o, c.os));
  s.lse = c.lse + ((int64_t)b * c.H + h0) * c.N;
  s.seg = c.seg + (int64_t)b * c.N;
  s.time = c.time + (int64_t)b * c.N;
  s.pic = c.pic ? c.pic + (int64_t)b * c.N : nullptr;
  s.mask = c.mask ? c.mask + (int64_t)b * c.N : nullptr;   // planes stay c.mask_plane apart
  s.B = 1;
  s.H = hc;
  return s;
}

int enqueue_call(const Call& c, char* ws, bool run_meta, bool debug, hipStream_t stream, tara_run_info_t* out) {
  const tara_params_t* p = c.p;
  const tara_dtype_t dtype = c.dtype;
  const int B = c.B, H = c.H, N = c.N, D = c.D;
  const void *q = c.q, *k = c.k, *v = c.v;
  void* o = c.o;
  float* lse = c.lse;
  const int64_t *q_str = c.qs, *k_str = c.ks, *v_str = c.vs, *o_str = c.os;
  const uint8_t* seg_type = c.seg;
  const float* token_time = c.time;
  const int16_t* picture_id = c.pic;
  const float* mask_weight = c.mask;
  const TailSplit tail = call_tail(c);
  const WsLayout L = ws_layout_for(dtype, B, H, N, D, p, tail);

  // derived constants, in double then rounded once to fp32
  const double log2e = 1.4426950408889634;
  const double scale = p->softmax_scale > 0.0f ? (double)p->softmax_scale : 1.0 / std::sqrt((double)D);
  const bool bias_active = p->strength > 0.0f && p->cap > 0.0f;
  const int nbind = num_bindings(p);
  bool binding_active = false;
  if (p->binding_enabled)
    for (int j = 0; j < nbind; ++j)
      for (int i = 0; i < p->num_pictures; ++i) binding_active |= p->picture_gain[j][i] != 1.0f;

  const int parts = num_parts(p);
  const int npad = npad_of(N), nkt = npad / kBlockK;

  MetaArgs ma{};
  ma.seg = seg_type;
  ma.time = token_time;
  ma.pic = picture_id;
  ma.mask = mask_weight;
  ma.mask_plane = c.mask_plane;
  ma.B = B;
  ma.N = N;
  ma.npad = npad;
  ma.nkt = nkt;
  ma.bias_active = bias_active;
  ma.binding_active = binding_active;
  ma.num_pictures = table_pictures(p);
  ma.nbind = nbind;
  for (int j = 0; j < kMaxBindings; ++j)
    for (int i = 0; i < kMaxPictures; ++i)
      ma.lg2gain[j][i] = (binding_active && j < nbind && i < p->num_pictures)
                             ? (float)std::log2((double)p->picture_gain[j][i]) : 0.0f;
  ma.tq = reinterpret_cast<float*>(ws + L.tq);
  ma.tk = reinterpret_cast<float*>(ws + L.tk);
  ma.kp = reinterpret_cast<int*>(ws + L.kp);
  ma.gt = reinterpret_cast<float*>(ws + L.gt);
  ma.ksum = reinterpret_cast<KeyTileSummary*>(ws + L.ksum);

  AttnArgs aa{};
  aa.q = q;
  aa.k = k;
  aa.v = v;
  aa.vt = dtype == TARA_BF16 ? reinterpret_cast<const __bf16*>(ws + L.vt) : nullptr;
  aa.q_sb = q_str[0]; aa.q_sh = q_str[1]; aa.q_sn = q_str[2];
  aa.k_sb = k_str[0]; aa.k_sh = k_str[1]; aa.k_sn = k_str[2];
  aa.v_sb = v_str[0]; aa.v_sh = v_str[1]; aa.v_sn = v_str[2];
  aa.o_sb = o_str[0]; aa.o_sh = o_str[1]; aa.o_sn = o_str[2];
  aa.o = o;
  aa.lse = lse;
  // per-partition outputs: every mode but fused (range partitions, the three terms)
  aa.opart = has_partials(p) || tail.parts ? reinterpret_cast<float*>(ws + L.opart) : nullptr;
  aa.lsepart = has_partials(p) || tail.parts ? reinterpret_cast<float*>(ws + L.lsepart) : nullptr;
  aa.prow0 = 0;
  aa.prows = N;
  aa.B = B;
  aa.H = H;
  aa.N = N;
  aa.npad = npad;
  aa.nkt = nkt;
  aa.tq = ma.tq;
  aa.tk = ma.tk;
  aa.kp = ma.kp;
  aa.gt = ma.gt;
  aa.npics = ma.num_pictures;
  aa.ksum = ma.ksum;
  aa.kmax = dtype == TARA_BF16 ? reinterpret_cast<const float*>(ws + L.kmax) : nullptr;
  const bool qk8 = uses_qk8(dtype, p);
  aa.k8 = qk8 ? reinterpret_cast<const uint8_t*>(ws + L.k8) : nullptr;
  aa.ks = qk8 ? reinterpret_cast<const float*>(ws + L.ks) : nullptr;
  aa.c = (float)(scale * log2e);
  const double sigma = bias_active ? std::sqrt((double)p->strength * log2e) / (double)p->falloff : 0.0;
  aa.sigma = (float)sigma;
  aa.w = (float)((double)p->window * sigma);
  aa.cap2 = bias_active ? (float)((double)p->cap * log2e) : 0.0f;
  aa.window = p->window;
  aa.dsat = bias_active ? (float)((double)p->window + (double)p->falloff * std::sqrt((double)p->cap / (double)p->strength))
                        : INFINITY;
  aa.corr0 = bias_active ? (float)std::log2(-std::expm1(-(double)p->cap)) : -INFINITY;
  // TARA_DISABLE_TILE_SKIP=1: every key tile takes the per-element bias (the
  // tile classes are switched off; the results are the same up to rounding)
  aa.elem_all = env_flag("TARA_DISABLE_TILE_SKIP") ? 1 : 0;
  aa.nparts = parts;
  if (p->mode == TARA_MODE_PARTITIONED && p->partition_bounds) {
    for (int i = 0; i <= parts; ++i) aa.kr[i] = p->partition_bounds[i];
  } else {
    for (int i = 0; i <= parts; ++i) aa.kr[i] = (int)((int64_t)N * i / parts);
  }
  const bool partitioned = has_partials(p);
  aa.qr0 = 0;
  aa.qr1 = N;
  // query ranges, each its own launch of every pass (FRAME_LOOP: the caller's
  // ranges; otherwise all rows at once)
  std::vector<std::pair<int, int>> qranges;
  if (p->mode == TARA_MODE_FRAME_LOOP) {
    const int nr = p->num_partitions;
    for (int i = 0; i < nr; ++i) {
      const int r0 = p->partition_bounds ? p->partition_bounds[i] : (int)((int64_t)N * i / nr);
      const int r1 = p->partition_bounds ? p->partition_bounds[i + 1] : (int)((int64_t)N * (i + 1) / nr);
      if (r1 > r0) qranges.emplace_back(r0, r1);
    }
  } else {
    // a fused call with a tail split: the fused pass over the first rows only
    qranges.emplace_back(0, tail.parts ? tail.row0 : N);
  }
  // passes of the attention kernel: one fused pass, one pass over all key
  // ranges, or the three terms
  std::vector<int> passes;
  if (p->mode == TARA_MODE_PARTITIONED) passes = {PASS_RANGE};
  else if (p->mode == TARA_MODE_THREE_TERM) passes = {PASS_TERM_A, PASS_TERM_B, PASS_TERM_C};
  else passes = {PASS_FUSED};
  const bool dense = p->mode == TARA_MODE_DENSE_BIAS;
  aa.dbias = dense ? reinterpret_cast<const float*>(ws + L.dbias) : nullptr;
  const int variant = qk8 ? ATTN_QK8 : dense ? ATTN_DENSE_BIAS : ATTN_PLAIN;
  int launches = 0;
  hipError_t e = hipSuccess;
  if (run_meta) {
    e = launch_meta(ma, stream);
    ++launches;
  }
  if (e == hipSuccess && dtype == TARA_BF16) {
    e = launch_vtranspose(static_cast<const __bf16*>(v), v_str[0], v_str[1], v_str[2],
                                const_cast<__bf16*>(aa.vt), B, H, N, npad, D, stream);
    ++launches;
    if (e == hipSuccess) {
      // max key norm per tile; with 8-bit Q.K the quantising kernel instead, which writes the FP8
      // keys, the tile scales and the norms of the rounded keys
      if (qk8)
        e = launch_kquant(static_cast<const __bf16*>(k), k_str[0], k_str[1], k_str[2],
                                const_cast<uint8_t*>(aa.k8), const_cast<float*>(aa.ks), const_cast<float*>(aa.kmax),
                                B, H, N, npad, nkt, D, stream);
      else
        e = launch_knorm(static_cast<const __bf16*>(k), k_str[0], k_str[1], k_str[2],
                               const_cast<float*>(aa.kmax), B, H, N, nkt, D, stream);
      ++launches;
    }
  }
  if (e == hipSuccess && dense) {
    // the dense-bias baseline: every bias value written out before the attention pass
    e = launch_dense_bias(aa, const_cast<float*>(aa.dbias), stream);
    ++launches;
  }
  if (e != hipSuccess) return fail(TARA_ERR_HIP, std::string("prologue launch: ") + hipGetErrorString(e));

  for (int pass : passes)
    if (pass != PASS_FUSED && (!aa.opart || !aa.lsepart))
      return fail(TARA_ERR_HIP, "internal: a partition pass without its partial-output buffers");
  hipEvent_t ev0 = nullptr, ev1 = nullptr;
  if (debug) {
    std::lock_guard<std::mutex> lk(g_tmu);
    if (g_timing) {
      if (hipEventCreate(&ev0) != hipSuccess || hipEventCreate(&ev1) != hipSuccess) {
        if (ev0) (void)hipEventDestroy(ev0);
        return fail(TARA_ERR_HIP, "hipEventCreate failed");
      }
      (void)hipEventRecord(ev0, stream);
    }
  }
  int grid = 0, block_q = 0;
  for (const auto& qrange : qranges) {
    aa.qr0 = qrange.first;
    aa.qr1 = qrange.second;
    for (int pass : passes) {
      if (dtype == TARA_BF16) {
        block_q = attn_bf16_block_q(D);
        aa.nqb = (aa.qr1 - aa.qr0 + block_q - 1) / block_q;
        grid += attn_bf16_grid(aa) * (pass == PASS_RANGE ? parts : 1);
        e = launch_attn_bf16(aa, D, pass, variant, stream);
      } else {
        block_q = attn_f32_block_q(D);
        aa.nqb = (aa.qr1 - aa.qr0 + block_q - 1) / block_q;
        grid += aa.nqb * B * H * (pass == PASS_RANGE ? parts : 1);
        e = launch_attn_f32(aa, D, pass, stream);
      }
      ++launches;
      if (e != hipSuccess) break;
    }
    if (e != hipSuccess) break;
  }
  if (e == hipSuccess && tail.parts) {
    // the split-off rows [row0, N): the range pass over `parts` tile-aligned
    // key ranges, then their exact merge (inside the timed region: it is part
    // of the attention work)
    aa.qr0 = tail.row0;
    aa.qr1 = N;
    aa.nqb = (N - tail.row0 + block_q - 1) / block_q;
    aa.nparts = tail.parts;
    for (int i = 0; i <= tail.parts; ++i)
      aa.kr[i] = i == tail.parts ? N : (int)std::min<int64_t>(N, (int64_t)nkt * i / tail.parts * kBlockK);
    aa.prow0 = tail.row0;
    aa.prows = N - tail.row0;
    grid += attn_bf16_grid(aa) * tail.parts;
    e = launch_attn_bf16(aa, D, PASS_RANGE, variant, stream);
    ++launches;
    if (e == hipSuccess) {
      MergeArgs mg{};
      mg.opart = aa.opart;
      mg.lsepart = aa.lsepart;
      mg.o = o;
      mg.lse = lse;
      mg.o_sb = o_str[0]; mg.o_sh = o_str[1]; mg.o_sn = o_str[2];
      mg.B = B; mg.H = H; mg.N = N; mg.D = D; mg.nparts = tail.parts;
      mg.row0 = tail.row0;
      mg.rows = N - tail.row0;
      e = launch_merge(mg, true, stream);
      ++launches;
    }
  }
  if (ev1) {
    std::lock_guard<std::mutex> lk(g_tmu);
    (void)hipEventRecord(ev1, stream);
    g_events.emplace_back(ev0, ev1);
  }
  if (e != hipSuccess) return fail(TARA_ERR_HIP, std::string("attention launch: ") + hipGetErrorString(e));
  if (partitioned) {
    MergeArgs mg{};
    mg.opart = aa.opart;
    mg.lsepart = aa.lsepart;
    mg.o = o;
    mg.lse = lse;
    mg.o_sb = o_str[0]; mg.o_sh = o_str[1]; mg.o_sn = o_str[2];
    mg.B = B; mg.H = H; mg.N = N; mg.D = D; mg.nparts = parts;
    mg.row0 = 0;
    mg.rows = N;
    e = launch_merge(mg, dtype == TARA_BF16, stream);
    ++launches;
    if (e != hipSuccess) return fail(TARA_ERR_HIP, std::string("merge launch: ") + hipGetErrorString(e));
  }
  const int parts_info = p->mode == TARA_MODE_FRAME_LOOP ? (int)qranges.size() : parts;
  tara_run_info_t info{};
  info.mode = p->mode;
  info.dtype = (int)dtype;
  info.bias_active = bias_active;
  info.binding_active = binding_active;
  info.num_partitions = parts_info;
  info.block_q = block_q;
  info.block_k = kBlockK;
  info.grid = grid;
  info.launches = launches;
  info.elem_all = aa.elem_all;
  info.tail_parts = tail.parts;
  const bool log = env_flag("TARA_LOG");
  if (debug && (log || env_flag("TARA_TILE_STATS")) && dtype == TARA_BF16 &&
      (p->mode == TARA_MODE_FUSED || p->mode == TARA_MODE_PARTITIONED)) {
    // debug readback: replay the bias-class decisions and count them (synchronous)
    const int ng = tile_stats_groups(N);
    unsigned* dcounts = reinterpret_cast<unsigned*>(ws + L.tstats);
    std::vector<unsigned> hc((size_t)B * ng * TC_COUNT);
    e = launch_tile_stats(aa, partitioned ? PASS_RANGE : PASS_FUSED, dcounts, stream);
    if (e == hipSuccess) e = hipMemcpyAsync(hc.data(), dcounts, hc.size() * 4, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fail(TARA_ERR_HIP, std::string("tile statistics: ") + hipGetErrorString(e));
    long long t[TC_COUNT] = {};
    for (size_t i = 0; i < hc.size(); ++i) t[i % TC_COUNT] += hc[i];
    info.tile_stats = 1;
    info.tiles_plain = t[TC_PLAIN] * H;
    info.tiles_saturated = t[TC_SATURATED] * H;
    info.tiles_window = t[TC_WINDOW] * H;
    info.tiles_picture = t[TC_PICTURE] * H;
    info.tiles_elem = t[TC_ELEM] * H;
  }
  *out = info;
  if (log && debug) {
    std::fprintf(stderr, "[tara] %s %s B=%d H=%d N=%d D=%d bias=%d binding=%d parts=%d grid=%d launches=%d%s",
                 p->mode == TARA_MODE_THREE_TERM   ? "three-term"
                 : p->mode == TARA_MODE_DENSE_BIAS ? "dense-bias"
                 : p->mode == TARA_MODE_FRAME_LOOP ? "frame-loop"
                 : partitioned                     ? "partitioned"
                                                   : "fused",
                 dtype == TARA_BF16 ? "bf16" : "fp32", B, H, N, D,
                 (int)bias_active, (int)binding_active, parts_info, grid, launches,
                 aa.elem_all ? " tile-skip=off" : "");
    if (info.tile_stats)
      std::fprintf(stderr, " tiles plain=%lld saturated=%lld window=%lld picture=%lld elem=%lld",
                   info.tiles_plain, info.tiles_saturated, info.tiles_window, info.tiles_picture, info.tiles_elem);
    if (tail.parts)
      std::fprintf(stderr, " tail: rows %d.. over %d key ranges", tail.row0, tail.parts);
    std::fprintf(stderr, "\n");
  }
  return TARA_OK;
}

}  // namespace tara

extern "C" {

void tara_params_default(tara_params_t* p) {
  if (!p) return;
  std::memset(p, 0, sizeof(*p));
  p->window = 0.20f;
  p->falloff = 0.25f;
  p->strength = 2.0f;
  p->cap = 6.0f;
  p->binding_enabled = 0;
  p->num_pictures = 0;
  p->num_bindings = 1;
  for (int j = 0; j < TARA_MAX_BINDINGS; ++j)
    for (int i = 0; i < TARA_MAX_PICTURES; ++i) p->picture_gain[j][i] = 1.0f;
  p->softmax_scale = 0.0f;
  p->mode = TARA_MODE_FUSED;
  p->num_partitions = 1;
  p->partition_bounds = nullptr;
}

size_t tara_workspace_bytes(int dtype_, int B, int H, int N, int D, const tara_params_t* p) {
  if (!p || (dtype_ != TARA_BF16 && dtype_ != TARA_FP32) || (D != 64 && D != 128)) return (size_t)-1;
  const tara_dtype_t dtype = (tara_dtype_t)dtype_;
  if (B < 0 || H < 0 || N < 0) return (size_t)-1;
  if (p->mode == TARA_MODE_PARTITIONED && (p->num_partitions < 1 || p->num_partitions > TARA_MAX_PARTITIONS))
    return (size_t)-1;
  if (!qk8_supported(dtype, p)) return (size_t)-1;
  if (p->mode == TARA_MODE_DENSE_BIAS && dtype != TARA_BF16) return (size_t)-1;
  if (B == 0 || H == 0 || N == 0) return 0;
  return ws_layout_for(dtype, B, H, N, D, p, tail_split(dtype, B, H, N, D, p)).total;
}

const char* tara_status_string(int status) {
  switch (status) {
    case TARA_OK: return "ok";
    case TARA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case TARA_ERR_BAD_SHAPE: return "bad shape (B, H or N)";
    case TARA_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype";
    case TARA_ERR_UNSUPPORTED_HEAD_DIM: return "unsupported head dim (64 or 128)";
    case TARA_ERR_BAD_STRIDE: return "bad stride or alignment";
    case TARA_ERR_BAD_PARAM: return "bad parameter";
    case TARA_ERR_WORKSPACE: return "workspace missing or too small";
    case TARA_ERR_BAD_METADATA: return "metadata out of range";
    case TARA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* tara_last_error(void) { return g_err.c_str(); }

int tara_get_last_run_info(tara_run_info_t* info) {
  if (!info) return fail(TARA_ERR_NULL_POINTER, "info is NULL");
  if (!g_info_valid) std::memset(info, 0, sizeof(*info));
  else *info = g_info;
  return TARA_OK;
}

int tara_timing_enable(int on) {
  std::lock_guard<std::mutex> lk(g_tmu);
  g_timing = on != 0;
  return TARA_OK;
}

int tara_timing_read(float* ms_out, int max, int* count) {
  if (!count || (max > 0 && !ms_out)) return fail(TARA_ERR_NULL_POINTER, "ms_out/count is NULL");
  std::lock_guard<std::mutex> lk(g_tmu);
  int n = 0;
  int status = TARA_OK;
  for (auto& ev : g_events) {
    float ms = 0.0f;
    if (hipEventSynchronize(ev.second) != hipSuccess || hipEventElapsedTime(&ms, ev.first, ev.second) != hipSuccess)
      status = fail(TARA_ERR_HIP, "hipEventElapsedTime failed");
    else if (n < max)
      ms_out[n++] = ms;
    (void)hipEventDestroy(ev.first);
    (void)hipEventDestroy(ev.second);
  }
  g_events.clear();
  *count = n;
  return status;
}

int tara_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int dtype,
                  int B, int H, int N, int D, const int64_t q_str[3], const int64_t k_str[3],
                  const int64_t v_str[3], const int64_t o_str[3], const uint8_t* seg_type,
                  const float* token_time, const int16_t* picture_id, const float* mask_weight,
                  const tara_params_t* p, void* workspace, size_t workspace_bytes, tara_stream_t stream_) {
  g_err.clear();
  hipStream_t stream = reinterpret_cast<hipStream_t>(stream_);
  tara::Call c{};
  if (int st = tara::make_call(c, q, k, v, o, lse, dtype, B, H, N, D, q_str, k_str, v_str, o_str, seg_type,
                               token_time, picture_id, mask_weight, p))
    return st;
  if (B == 0 || H == 0 || N == 0) {
    tara::set_empty_info(c);
    return TARA_OK;
  }
  const size_t need = tara::call_workspace(c);
  if (!workspace) return fail(TARA_ERR_WORKSPACE, "workspace is NULL");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return fail(TARA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (workspace_bytes < need)
    return fail(TARA_ERR_WORKSPACE, "workspace needs " + std::to_string(need) + " bytes, got " +
                                        std::to_string(workspace_bytes));
  if (env_flag("TARA_VALIDATE"))
    if (int st = validate_metadata(B, N, seg_type, token_time, picture_id, mask_weight, p, stream)) return st;
  tara_run_info_t info{};
  if (int st = tara::enqueue_call(c, static_cast<char*>(workspace), true, true, stream, &info)) return st;
  tara::set_last_info(info);
  return TARA_OK;
}

}  // extern "C"
