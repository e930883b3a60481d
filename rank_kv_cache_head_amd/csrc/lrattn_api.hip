// C-ABI host layer of liblrattn: argument validation, the partition plan,
// workspace sizing and kernel launches.  Every argument error is detected here,
// on the host, before any HIP call, so a rejected call has no device effect.
#include <math.h>
#include <initializer_list>
#include <stdint.h>
#include <string.h>

#include "lrattn.h"
#include "lrattn_append.hpp"
#include "lrattn_internal.hpp"
#include "lrattn_shared.hpp"
#include "lrattn_probe.h"

namespace {

using lrattn::kRecPad;

constexpr int kVersion = 10000;  // 1.0.0

// Default partition plan (num_splits = 0), from measurements on MI355X:
// a partition streams at least kSplitBytes of latents (and scales) and at
// least kSplitTokensPerHead tokens per query head of its group, since each
// workgroup pays a fixed prologue (absorbing q into the factor) and epilogue
// (merging its waves); the split is only made finer when that would leave
// fewer than kMinBlocks workgroups.
constexpr int64_t kSplitBytes = 128 * 1024;
constexpr int64_t kSplitTokensPerHead = 1024;
constexpr int64_t kMinBlocks = 512;
constexpr int64_t kMinSplitTokens = 256;

int esize(int dt) {
  switch (dt) {
    case LRATTN_F32: return 4;
    case LRATTN_BF16: case LRATTN_F16: return 2;
    case LRATTN_I8: return 1;
    default: return 0;
  }
}

bool is_float_dtype(int dt) { return dt == LRATTN_F32 || dt == LRATTN_BF16 || dt == LRATTN_F16; }

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// Product of positive factors, or -1 when it would pass 2^62.
int64_t checked_mul(std::initializer_list<int64_t> xs) {
  int64_t r = 1;
  for (int64_t x : xs) {
    if (x <= 0) return -1;
    if (r > (int64_t(1) << 62) / x) return -1;
    r *= x;
  }
  return r;
}

struct Plan {
  int32_t P;  // partitions per (b, kv-head)
  int32_t S;  // tokens per partition
};

// Validates the parameter block alone (no pointers).
int check_params(const lrattn_params* p, Plan* plan) {
  if (!p) return LRATTN_ERR_NULL;
  if (p->batch <= 0 || p->num_q_heads <= 0 || p->num_kv_heads <= 0 || p->head_dim <= 0 ||
      p->rank <= 0 || p->max_seq_len <= 0)
    return LRATTN_ERR_SHAPE;
  if (p->num_q_heads % p->num_kv_heads) return LRATTN_ERR_SHAPE;
  if (!is_float_dtype(p->q_dtype) || esize(p->latent_dtype) == 0 ||
      !is_float_dtype(p->factor_dtype) ||
      (p->out_dtype != LRATTN_F32 && p->out_dtype != LRATTN_BF16))
    return LRATTN_ERR_DTYPE;
  if (checked_mul({p->batch, p->num_kv_heads, p->max_seq_len, p->rank, 4}) < 0 ||
      checked_mul({p->batch, p->num_q_heads, p->head_dim, 4}) < 0)
    return LRATTN_ERR_SHAPE;
  if (!(isfinite(p->softmax_scale))) return LRATTN_ERR_SHAPE;
  const int group = p->num_q_heads / p->num_kv_heads;
  const int d = p->head_dim;
  if (!(d == 64 || d == 128 || d == 256)) return LRATTN_ERR_UNSUPPORTED;
  if (!lrattn::partition_supported(p->latent_dtype, p->rank, group)) return LRATTN_ERR_UNSUPPORTED;
  if (p->batch > 65535 || p->num_kv_heads > 65535) return LRATTN_ERR_UNSUPPORTED;
  if (p->num_splits < 0 || p->num_splits > p->max_seq_len) return LRATTN_ERR_SPLITS;

  const int64_t T = p->max_seq_len;
  int64_t splits = p->num_splits;
  if (splits == 0) {
    const int64_t pairs = (int64_t)p->batch * p->num_kv_heads;
    const int64_t row_pair = 2 * (int64_t)p->rank * esize(p->latent_dtype) +
                             (p->latent_dtype == LRATTN_I8 ? 8 : 0);
    int64_t tokens = (kSplitBytes + row_pair - 1) / row_pair;
    if (tokens < kSplitTokensPerHead * group) tokens = kSplitTokensPerHead * group;
    tokens = (tokens + 255) / 256 * 256;
    splits = (T + tokens - 1) / tokens;
    if (pairs * splits < kMinBlocks) {
      const int64_t cap = (T + kMinSplitTokens - 1) / kMinSplitTokens;
      const int64_t want = (kMinBlocks + pairs - 1) / pairs;
      splits = want < cap ? want : cap;
    }
    if (splits < 1) splits = 1;
  }
  const int64_t S = (T + splits - 1) / splits;
  const int64_t P = (T + S - 1) / S;
  // byte offsets inside one partition stay below 2^30 (buffer addressing)
  if (S * p->rank * esize(p->latent_dtype) >= (int64_t(1) << 30)) return LRATTN_ERR_UNSUPPORTED;
  if (P > 2147483647LL) return LRATTN_ERR_UNSUPPORTED;
  if (checked_mul({p->batch, p->num_q_heads, P, p->rank + kRecPad, 4}) < 0) return LRATTN_ERR_SHAPE;
  if (plan) { plan->P = (int32_t)P; plan->S = (int32_t)S; }
  return LRATTN_OK;
}

size_t workspace_bytes_for(const lrattn_params* p, const Plan& pl) {
  return lrattn::records_bytes(p->batch, p->num_q_heads, pl.P, p->rank);
}

// With many partitions per head, the decode step absorbs q . B_K^T once per
// query head in a small kernel ahead of the partition kernel, instead of once
// per partition in each workgroup's prologue; the absorbed queries [B, Hq, r]
// fp32 follow the records in the workspace.  Measured on MI355X at 256
// partitions per head (4 x 40 heads, r 48, up to 131072 tokens): the step
// 237.9 -> 235.2 us; with 4 partitions per head the extra launch costs ~4 us
// (gqa_vlm 87.8 -> 92.0 us), hence the threshold.
bool pre_absorb(const Plan& pl) { return pl.P >= LRATTN_PRE_ABSORB_SPLITS; }

size_t decode_workspace_bytes(const lrattn_params* p, const Plan& pl) {
  size_t b = workspace_bytes_for(p, pl);
  if (pre_absorb(pl)) b += ((size_t)p->batch * p->num_q_heads * p->rank * 4 + 255) & ~(size_t)255;
  return b;
}

float qscale_for(const lrattn_params* p) {
  const float scale = p->softmax_scale > 0.f ? p->softmax_scale
                                             : (float)(1.0 / sqrt((double)p->head_dim));
  return (float)((double)scale * 1.4426950408889634);  // log2(e): logits in base 2
}

// Launches absorb_heads_kernel into the workspace's q~ area and points the
// partition arguments at it, when the plan asks for it.
int launch_pre_absorb(const lrattn_params* p, const Plan& pl, const void* q, const void* BK,
                      void* ws, lrattn::PartitionArgs* pa, hipStream_t s) {
  if (!pre_absorb(pl)) return LRATTN_OK;
  float* qt = reinterpret_cast<float*>(static_cast<char*>(ws) + workspace_bytes_for(p, pl));
  lrattn::AbsorbHeadsArgs ab;
  ab.q = q; ab.BK = BK; ab.qt = qt;
  ab.B = p->batch; ab.Hq = p->num_q_heads; ab.d = p->head_dim; ab.r = p->rank;
  ab.hpf = p->num_q_heads / p->num_kv_heads;
  ab.q_dtype = p->q_dtype; ab.f_dtype = p->factor_dtype; ab.qscale = qscale_for(p);
  if (lrattn::launch_absorb_heads(ab, s) != hipSuccess) return LRATTN_ERR_HIP;
  pa->qt_pre = qt;
  return LRATTN_OK;
}

int check_workspace(const lrattn_params* p, const Plan& pl, const void* ws, size_t ws_bytes,
                    size_t need = 0) {
  if (!ws) return LRATTN_ERR_WORKSPACE;
  if (!aligned16(ws)) return LRATTN_ERR_ALIGN;
  if (ws_bytes < (need ? need : workspace_bytes_for(p, pl))) return LRATTN_ERR_WORKSPACE;
  return LRATTN_OK;
}

int check_partition_ptrs(const lrattn_params* p, const void* q, const void* LK, const void* LV,
                         const void* BK, const float* scales, const int32_t* seq_lens) {
  if (!q || !LK || !LV || !BK || !seq_lens) return LRATTN_ERR_NULL;
  const bool int8 = p->latent_dtype == LRATTN_I8;
  if (int8 != (scales != nullptr)) return LRATTN_ERR_NULL;
  if (!aligned16(q) || !aligned16(LK) || !aligned16(LV) || !aligned16(BK) ||
      !aligned16(seq_lens) || (scales && !aligned16(scales)))
    return LRATTN_ERR_ALIGN;
  return LRATTN_OK;
}

int check_combine_ptrs(const void* BV, const int32_t* seq_lens, const void* out) {
  if (!BV || !seq_lens || !out) return LRATTN_ERR_NULL;
  if (!aligned16(BV) || !aligned16(seq_lens) || !aligned16(out)) return LRATTN_ERR_ALIGN;
  return LRATTN_OK;
}

lrattn::MergeArgs merge_args(const lrattn_params* p, const void* BV, void* out) {
  lrattn::MergeArgs m;
  m.BV = BV; m.out = out; m.f_dtype = p->factor_dtype; m.out_dtype = p->out_dtype;
  return m;
}

lrattn::PartitionArgs partition_args(const lrattn_params* p, const Plan& pl, const void* q,
                                     const void* LK, const void* LV, const void* BK,
                                     const float* scales, const int32_t* seq_lens, void* ws) {
  lrattn::PartitionArgs a;
  a.q = q; a.LK = LK; a.LV = LV; a.BK = BK; a.scales = scales; a.seq_lens = seq_lens;
  a.rope = nullptr;
  a.qt_pre = nullptr;
  a.ws = static_cast<float*>(ws);
  a.B = p->batch; a.Hq = p->num_q_heads; a.Hkv = p->num_kv_heads; a.d = p->head_dim;
  a.HG = p->num_kv_heads;                        // one group per kv-head
  a.hps = p->num_q_heads / p->num_kv_heads;
  a.xcd_group = 0;
  a.T = p->max_seq_len; a.P = pl.P; a.S = pl.S;
  a.t_lo = 0; a.t_hi = p->max_seq_len; a.p_off = 0; a.P_rec = pl.P;
  a.BK1 = nullptr; a.n_img = 0; a.P_img = 0; a.S_img = 1;
  a.imp = nullptr; a.logits = nullptr; a.imp_thr = 0.f; a.low_rank = p->rank;
  a.q_dtype = p->q_dtype; a.f_dtype = p->factor_dtype;
  a.qscale = qscale_for(p);
  return a;
}

lrattn::CombineArgs combine_args(const lrattn_params* p, const Plan& pl, const void* BV,
                                 const int32_t* seq_lens, void* out, void* ws) {
  lrattn::CombineArgs a;
  a.seq_lens = seq_lens; a.ws = static_cast<const float*>(ws); a.merge = merge_args(p, BV, out);
  a.B = p->batch; a.Hq = p->num_q_heads; a.Hkv = p->num_kv_heads; a.d = p->head_dim;
  a.r = p->rank; a.T = p->max_seq_len; a.P = pl.P; a.S = pl.S;
  a.factor_per_head = 0;
  a.BV1 = nullptr; a.n_img = 0; a.P_img = 0; a.S_img = 1;
  a.stats = nullptr;
  return a;
}

int group_of(const lrattn_params* p) { return p->num_q_heads / p->num_kv_heads; }

}  // namespace

extern "C" {

int lrattn_version(void) { return kVersion; }

const char* lrattn_status_string(int status) {
  switch (status) {
    case LRATTN_OK: return "ok";
    case LRATTN_ERR_NULL: return "null pointer (or scales given for non-int8 latents)";
    case LRATTN_ERR_SHAPE: return "invalid shape";
    case LRATTN_ERR_DTYPE: return "invalid dtype";
    case LRATTN_ERR_UNSUPPORTED: return "unsupported shape/dtype combination";
    case LRATTN_ERR_ALIGN: return "pointer not 16-byte aligned";
    case LRATTN_ERR_WORKSPACE: return "workspace missing or too small";
    case LRATTN_ERR_SPLITS: return "num_splits out of range";
    case LRATTN_ERR_HIP: return "HIP launch failed";
    case LRATTN_ERR_SCRATCH: return "records exceed the static scratch buffer (LRATTN_STATIC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

int lrattn_plan(const lrattn_params* p, int32_t* num_splits, int32_t* split_tokens) {
  Plan pl;
  const int st = check_params(p, &pl);
  if (st != LRATTN_OK) return st;
  if (num_splits) *num_splits = pl.P;
  if (split_tokens) *split_tokens = pl.S;
  return LRATTN_OK;
}

const char* lrattn_partition_kernel(const lrattn_params* p) {
  Plan pl;
  if (check_params(p, &pl) != LRATTN_OK) return nullptr;
  return lrattn::partition_kernel_name(p->latent_dtype, p->rank, group_of(p));
}

int lrattn_workspace_size(const lrattn_params* p, size_t* bytes) {
  if (!bytes) return LRATTN_ERR_NULL;
  Plan pl;
  const int st = check_params(p, &pl);
  if (st != LRATTN_OK) return st;
  *bytes = decode_workspace_bytes(p, pl);
  return LRATTN_OK;
}

int lrattn_partition(const lrattn_params* p, const void* q, const void* L_K, const void* L_V,
                     const void* B_K, const float* scales, const int32_t* seq_lens,
                     void* workspace, size_t workspace_bytes, lrattn_stream stream) {
  Plan pl;
  int st = check_params(p, &pl);
  if (st == LRATTN_OK) st = check_partition_ptrs(p, q, L_K, L_V, B_K, scales, seq_lens);
  if (st == LRATTN_OK)
    st = check_workspace(p, pl, workspace, workspace_bytes, decode_workspace_bytes(p, pl));
  if (st != LRATTN_OK) return st;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  auto a = partition_args(p, pl, q, L_K, L_V, B_K, scales, seq_lens, workspace);
  st = launch_pre_absorb(p, pl, q, B_K, workspace, &a, s);
  if (st != LRATTN_OK) return st;
  if (lrattn::launch_partition(p->latent_dtype, p->rank, group_of(p), a, s) != hipSuccess)
    return LRATTN_ERR_HIP;
  return LRATTN_OK;
}

int lrattn_combine(const lrattn_params* p, const void* B_V, const int32_t* seq_lens, void* out,
                   void* workspace, size_t workspace_bytes, lrattn_stream stream) {
  Plan pl;
  int st = check_params(p, &pl);
  if (st == LRATTN_OK) st = check_combine_ptrs(B_V, seq_lens, out);
  if (st == LRATTN_OK) st = check_workspace(p, pl, workspace, workspace_bytes);
  if (st != LRATTN_OK) return st;
  const auto a = combine_args(p, pl, B_V, seq_lens, out, workspace);
  if (lrattn::launch_combine(group_of(p), a, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return LRATTN_ERR_HIP;
  return LRATTN_OK;
}

int lrattn_decode(const lrattn_params* p, const void* q, const void* L_K, const void* L_V,
                  const void* B_K, const void* B_V, const float* scales, const int32_t* seq_lens,
                  void* out, void* workspace, size_t workspace_bytes, lrattn_stream stream) {
  Plan pl;
  int st = check_params(p, &pl);
  if (st == LRATTN_OK) st = check_partition_ptrs(p, q, L_K, L_V, B_K, scales, seq_lens);
  if (st == LRATTN_OK) st = check_combine_ptrs(B_V, seq_lens, out);
  if (st == LRATTN_OK)
    st = check_workspace(p, pl, workspace, workspace_bytes, decode_workspace_bytes(p, pl));
  if (st != LRATTN_OK) return st;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  auto pa = partition_args(p, pl, q, L_K, L_V, B_K, scales, seq_lens, workspace);
  st = launch_pre_absorb(p, pl, q, B_K, workspace, &pa, s);
  if (st != LRATTN_OK) return st;
  if (lrattn::launch_partition(p->latent_dtype, p->rank, group_of(p), pa, s) != hipSuccess)
    return LRATTN_ERR_HIP;
  const auto ca = combine_args(p, pl, B_V, seq_lens, out, workspace);
  if (lrattn::launch_combine(group_of(p), ca, s) != hipSuccess) return LRATTN_ERR_HIP;
  return LRATTN_OK;
}

int lrattn_dense_decode(const lrattn_params* p, const void* q, const void* K, const void* V,
                        const float* scales, const int32_t* seq_lens, void* out,
                        void* workspace, size_t workspace_bytes, lrattn_stream stream) {
  Plan pl;
  int st = check_params(p, &pl);
  if (st == LRATTN_OK && p->rank != p->head_dim) st = LRATTN_ERR_SHAPE;
  if (st == LRATTN_OK && (!q || !K || !V || !seq_lens || !out)) st = LRATTN_ERR_NULL;
  if (st == LRATTN_OK && (p->latent_dtype == LRATTN_I8) != (scales != nullptr)) st = LRATTN_ERR_NULL;
  if (st == LRATTN_OK && (!aligned16(q) || !aligned16(K) || !aligned16(V) || !aligned16(seq_lens) ||
                          !aligned16(out) || (scales && !aligned16(scales))))
    st = LRATTN_ERR_ALIGN;
  if (st == LRATTN_OK) st = check_workspace(p, pl, workspace, workspace_bytes);
  if (st != LRATTN_OK) return st;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // no factors: the kernels take q~ = scale * q and write v~ as the output
  const auto pa = partition_args(p, pl, q, K, V, nullptr, scales, seq_lens, workspace);
  if (lrattn::launch_partition(p->latent_dtype, p->rank, group_of(p), pa, s) != hipSuccess)
    return LRATTN_ERR_HIP;
  const auto ca = combine_args(p, pl, nullptr, seq_lens, out, workspace);
  if (lrattn::launch_combine(group_of(p), ca, s) != hipSuccess) return LRATTN_ERR_HIP;
  return LRATTN_OK;
}

namespace {
// Attention-aware rank: the decode plan's records, then the step's base-2
// logits [B, Hkv, T, Hq / Hkv] and each row's final (max, denominator) [B, Hq, 2], each
// part at a 256-byte boundary.
int adaptive_check(const lrattn_params* p, const lrattn_adaptive* ad, Plan* pl,
                   size_t* logits_off, size_t* stats_off, size_t* total) {
  int st = check_params(p, pl);
  if (st != LRATTN_OK) return st;
  if (!ad) return LRATTN_ERR_NULL;
  if (ad->low_rank < 1 || ad->low_rank > p->rank || !(ad->decay >= 0.f && ad->decay <= 1.f) ||
      isnan(ad->threshold))
    return LRATTN_ERR_SHAPE;
  if (!lrattn::adaptive_supported(p->latent_dtype, p->rank, group_of(p)))
    return LRATTN_ERR_UNSUPPORTED;
  if (checked_mul({p->batch, p->num_q_heads, p->max_seq_len, 4}) < 0) return LRATTN_ERR_SHAPE;
  // a partition's logits are addressed with 32-bit offsets
  if ((int64_t)group_of(p) * p->max_seq_len * 4 >= (int64_t(1) << 31)) return LRATTN_ERR_UNSUPPORTED;
  const size_t rec = workspace_bytes_for(p, *pl);
  const size_t lg = ((size_t)p->batch * p->num_q_heads * p->max_seq_len * 4 + 255) & ~(size_t)255;
  *logits_off = rec;
  *stats_off = rec + lg;
  *total = rec + lg + (((size_t)p->batch * p->num_q_heads * 8 + 255) & ~(size_t)255);
  return LRATTN_OK;
}
}  // namespace

int lrattn_adaptive_workspace_size(const lrattn_params* p, const lrattn_adaptive* ad,
                                   size_t* bytes) {
  if (!bytes) return LRATTN_ERR_NULL;
  Plan pl;
  size_t lo, so, total;
  const int st = adaptive_check(p, ad, &pl, &lo, &so, &total);
  if (st != LRATTN_OK) return st;
  *bytes = total;
  return LRATTN_OK;
}

const char* lrattn_adaptive_kernel(const lrattn_params* p, const lrattn_adaptive* ad) {
  Plan pl;
  size_t lo, so, total;
  if (adaptive_check(p, ad, &pl, &lo, &so, &total) != LRATTN_OK) return nullptr;
  return lrattn::adaptive_kernel_name(p->latent_dtype, p->rank, group_of(p));
}

int lrattn_adaptive_decode(const lrattn_params* p, const lrattn_adaptive* ad, const void* q,
                           const void* L_K, const void* L_V, const void* B_K, const void* B_V,
                           const float* scales, const int32_t* seq_lens, float* importance,
                           void* out, void* workspace, size_t workspace_bytes,
                           lrattn_stream stream) {
  Plan pl;
  size_t lo = 0, so = 0, total = 0;
  int st = adaptive_check(p, ad, &pl, &lo, &so, &total);
  if (st == LRATTN_OK) st = check_partition_ptrs(p, q, L_K, L_V, B_K, scales, seq_lens);
  if (st == LRATTN_OK) st = check_combine_ptrs(B_V, seq_lens, out);
  if (st == LRATTN_OK && !importance) st = LRATTN_ERR_NULL;
  if (st == LRATTN_OK && !aligned16(importance)) st = LRATTN_ERR_ALIGN;
  if (st == LRATTN_OK) st = check_workspace(p, pl, workspace, workspace_bytes);
  if (st == LRATTN_OK && workspace_bytes < total) st = LRATTN_ERR_WORKSPACE;
  if (st != LRATTN_OK) return st;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  float* logits = reinterpret_cast<float*>(static_cast<char*>(workspace) + lo);
  float* stats = reinterpret_cast<float*>(static_cast<char*>(workspace) + so);
  auto pa = partition_args(p, pl, q, L_K, L_V, B_K, scales, seq_lens, workspace);
  pa.imp = importance;
  pa.logits = logits;
  pa.imp_thr = ad->threshold;
  pa.low_rank = ad->low_rank;
  if (lrattn::launch_adaptive(p->latent_dtype, p->rank, group_of(p), pa, s) != hipSuccess)
    return LRATTN_ERR_HIP;
  auto ca = combine_args(p, pl, B_V, seq_lens, out, workspace);
  ca.stats = stats;
  if (lrattn::launch_combine(group_of(p), ca, s) != hipSuccess) return LRATTN_ERR_HIP;
  lrattn::ImportanceArgs ia;
  ia.logits = logits; ia.stats = stats; ia.imp = importance; ia.seq_lens = seq_lens;
  ia.B = p->batch; ia.Hq = p->num_q_heads; ia.Hkv = p->num_kv_heads; ia.T = p->max_seq_len;
  ia.decay = ad->decay;
  if (lrattn::launch_importance(ia, s) != hipSuccess) return LRATTN_ERR_HIP;
  return LRATTN_OK;
}

namespace {
// Image block, then text (AttentionPack page, section 2.A: the modalities are
// compressed apart, each with its own factors).  Tokens [0, ni) and [ni, T)
// are planned apart, each in parts of at most the decode plan's S, so that no
// partition mixes the two factor sets: records [0, P_img) hold the image
// parts, [P_img, P_img + P_txt) the text parts.
struct ModalPlan {
  int32_t ni, P_img, S_img, P_txt, S_txt;
};

int modal_plan(const lrattn_params* p, int32_t image_tokens, Plan* pl, ModalPlan* mp) {
  int st = check_params(p, pl);
  if (st != LRATTN_OK) return st;
  if (image_tokens < 0) return LRATTN_ERR_SHAPE;
  if (!lrattn::modal_supported(p->head_dim, p->rank)) return LRATTN_ERR_UNSUPPORTED;
  const int64_t T = p->max_seq_len, S = pl->S;
  const int64_t ni = image_tokens < T ? image_tokens : T, nt = T - ni;
  const int64_t P_img = (ni + S - 1) / S, P_txt = (nt + S - 1) / S;
  mp->ni = (int32_t)ni;
  mp->P_img = (int32_t)P_img;
  mp->S_img = P_img ? (int32_t)((ni + P_img - 1) / P_img) : 1;
  mp->P_txt = (int32_t)P_txt;
  mp->S_txt = P_txt ? (int32_t)((nt + P_txt - 1) / P_txt) : 1;
  pl->P = (int32_t)(P_img + P_txt);
  if (pl->P > 65535) return LRATTN_ERR_UNSUPPORTED;  // grid z: partitions
  if (checked_mul({p->batch, p->num_q_heads, pl->P, p->rank + kRecPad, 4}) < 0)
    return LRATTN_ERR_SHAPE;
  return LRATTN_OK;
}
}  // namespace

int lrattn_modal_workspace_size(const lrattn_params* p, int32_t image_tokens, size_t* bytes) {
  if (!bytes) return LRATTN_ERR_NULL;
  Plan pl;
  ModalPlan mp;
  const int st = modal_plan(p, image_tokens, &pl, &mp);
  if (st != LRATTN_OK) return st;
  *bytes = workspace_bytes_for(p, pl);
  return LRATTN_OK;
}

int lrattn_modal_decode(const lrattn_params* p, int32_t image_tokens, const void* q,
                        const void* L_K, const void* L_V, const void* B_K, const void* B_V,
                        const float* scales, const int32_t* seq_lens, void* out,
                        void* workspace, size_t workspace_bytes, lrattn_stream stream) {
  Plan pl;
  ModalPlan mp;
  int st = modal_plan(p, image_tokens, &pl, &mp);
  if (st == LRATTN_OK) st = check_partition_ptrs(p, q, L_K, L_V, B_K, scales, seq_lens);
  if (st == LRATTN_OK) st = check_combine_ptrs(B_V, seq_lens, out);
  if (st == LRATTN_OK) st = check_workspace(p, pl, workspace, workspace_bytes);
  if (st != LRATTN_OK) return st;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // set 1 (text) follows set 0 (image) in B_K and B_V: [2, Hkv, r, d]
  const size_t fset = (size_t)p->num_kv_heads * p->rank * p->head_dim * esize(p->factor_dtype);
  // one launch over both segments: partitions [0, P_img) the image tokens
  // with set 0, the rest the text with set 1
  auto pa = partition_args(p, pl, q, L_K, L_V, B_K, scales, seq_lens, workspace);
  pa.S = mp.S_txt;
  pa.BK1 = static_cast<const char*>(B_K) + fset;
  pa.n_img = mp.ni; pa.P_img = mp.P_img; pa.S_img = mp.S_img;
  if (lrattn::launch_partition(p->latent_dtype, p->rank, group_of(p), pa, s) != hipSuccess)
    return LRATTN_ERR_HIP;
  auto ca = combine_args(p, pl, B_V, seq_lens, out, workspace);
  ca.S = mp.S_txt;
  ca.BV1 = static_cast<const char*>(B_V) + fset;
  ca.n_img = mp.ni; ca.P_img = mp.P_img; ca.S_img = mp.S_img;
  if (lrattn::launch_combine(group_of(p), ca, s) != hipSuccess) return LRATTN_ERR_HIP;
  return LRATTN_OK;
}

namespace {
// Rebuilt keys: each wave owns one sequence's partition, four sequences per
// workgroup, so the default plan splits T into enough partitions for the grid
// (partitions x kv-heads x quads of sequences) to give every CU about two
// workgroups (the kernel runs two per CU); a partition is a whole number of
// 32-token steps, at least
// kRebuildMinTokens.  An explicit num_splits is used as given.
constexpr int64_t kRebuildBlocks = 512;
constexpr int64_t kRebuildMinTokens = 128;

int rebuild_plan(const lrattn_params* p, Plan* pl) {
  int st = check_params(p, pl);
  if (st != LRATTN_OK) return st;
  if (p->q_dtype != LRATTN_BF16 || p->latent_dtype != LRATTN_BF16 ||
      p->factor_dtype != LRATTN_BF16 ||
      !lrattn::rebuild_supported(p->head_dim, p->rank, group_of(p)))
    return LRATTN_ERR_UNSUPPORTED;
  if (p->num_splits > 0) return LRATTN_OK;
  const int64_t T = p->max_seq_len;
  const int64_t cells = (int64_t)p->num_kv_heads * ((p->batch + 3) / 4);
  const int64_t want = (kRebuildBlocks + cells - 1) / cells;
  int64_t S = (T + want - 1) / want;
  S = (S + 31) / 32 * 32;
  if (S < kRebuildMinTokens) S = kRebuildMinTokens;
  if (S > T) S = T;
  if (S * p->rank * 2 >= (int64_t(1) << 30)) return LRATTN_ERR_UNSUPPORTED;
  pl->S = (int32_t)S;
  pl->P = (int32_t)((T + S - 1) / S);
  if (checked_mul({p->batch, p->num_q_heads, pl->P, p->rank + kRecPad, 4}) < 0)
    return LRATTN_ERR_SHAPE;
  return LRATTN_OK;
}
}  // namespace

int lrattn_rebuild_plan(const lrattn_params* p, int32_t* num_splits, int32_t* split_tokens) {
  Plan pl;
  const int st = rebuild_plan(p, &pl);
  if (st != LRATTN_OK) return st;
  if (num_splits) *num_splits = pl.P;
  if (split_tokens) *split_tokens = pl.S;
  return LRATTN_OK;
}

int lrattn_rebuild_workspace_size(const lrattn_params* p, size_t* bytes) {
  if (!bytes) return LRATTN_ERR_NULL;
  Plan pl;
  const int st = rebuild_plan(p, &pl);
  if (st != LRATTN_OK) return st;
  *bytes = workspace_bytes_for(p, pl);
  return LRATTN_OK;
}

int lrattn_rebuild_decode(const lrattn_params* p, const void* q, const void* L_K,
                          const void* L_V, const void* B_K, const void* B_V, const float* rope,
                          const int32_t* seq_lens, void* out, void* workspace,
                          size_t workspace_bytes, lrattn_stream stream) {
  Plan pl;
  int st = rebuild_plan(p, &pl);
  if (st == LRATTN_OK && rope && (int64_t)p->max_seq_len * p->head_dim * 4 >= (int64_t(1) << 31))
    st = LRATTN_ERR_UNSUPPORTED;
  if (st == LRATTN_OK) st = check_partition_ptrs(p, q, L_K, L_V, B_K, nullptr, seq_lens);
  if (st == LRATTN_OK) st = check_combine_ptrs(B_V, seq_lens, out);
  if (st == LRATTN_OK && rope && !aligned16(rope)) st = LRATTN_ERR_ALIGN;
  if (st == LRATTN_OK) st = check_workspace(p, pl, workspace, workspace_bytes);
  if (st != LRATTN_OK) return st;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  auto pa = partition_args(p, pl, q, L_K, L_V, B_K, nullptr, seq_lens, workspace);
  pa.rope = rope;
  if (lrattn::launch_rebuild(p->head_dim, p->rank, group_of(p), pa, s) != hipSuccess)
    return LRATTN_ERR_HIP;
  const auto ca = combine_args(p, pl, B_V, seq_lens, out, workspace);
  if (lrattn::launch_combine(group_of(p), ca, s) != hipSuccess) return LRATTN_ERR_HIP;
  return LRATTN_OK;
}

namespace {
// Shared latent streams: query heads run in groups of up to 8 that read the
// same stream; the plan is the grouped path's for that group size.
int shared_group(const lrattn_params* p) {
  const int hps = p->num_q_heads / p->num_kv_heads;
  for (int g : {8, 4, 2, 1})
    if (hps % g == 0) return g;
  return 1;
}

// One pass per stream (bf16 latents, r in {32, 64, 128}, at least 32 heads
// per stream): each workgroup reads a tile once for up to 64 heads, so the
// default plan splits T into enough partitions for the grid (partitions x
// streams x head groups x sequences) to give every CU about one
// workgroup, in whole 64-token steps.  An explicit num_splits is used as
// given.  *once tells whether that kernel runs.
constexpr int64_t kOnceBlocks = 256;

int check_shared(const lrattn_params* p, lrattn_params* grouped, Plan* pl, bool* once = nullptr) {
  if (!p) return LRATTN_ERR_NULL;
  if (p->num_kv_heads <= 0 || p->num_q_heads <= 0 || p->num_q_heads % p->num_kv_heads)
    return LRATTN_ERR_SHAPE;
  *grouped = *p;
  grouped->num_kv_heads = p->num_q_heads / shared_group(p);  // one "kv-head" per group
  const int st = check_params(grouped, pl);
  if (st != LRATTN_OK) return st;
  const int nh = p->num_q_heads / p->num_kv_heads;
  const bool one = lrattn::shared_once_supported(p->latent_dtype, p->rank, nh);
  if (once) *once = one;
  if (one && p->num_splits == 0) {
    const int64_t T = p->max_seq_len;
    const int gh = 16 * lrattn::shared_once_blocks(nh);  // heads per workgroup
    const int64_t cells = (int64_t)p->batch * p->num_kv_heads * ((nh + gh - 1) / gh);
    const int64_t want = (kOnceBlocks + cells - 1) / cells;
    int64_t S = (T + want - 1) / want;
    S = (S + 63) / 64 * 64;
    if (S > T) S = T;
    pl->S = (int32_t)S;
    pl->P = (int32_t)((T + S - 1) / S);
    if (checked_mul({p->batch, p->num_q_heads, pl->P, p->rank + kRecPad, 4}) < 0)
      return LRATTN_ERR_SHAPE;
  }
  return LRATTN_OK;
}

size_t shared_ws_bytes(const lrattn_params* p, const Plan& pl) {
  const size_t rec = lrattn::records_bytes(p->batch, p->num_q_heads, pl.P, p->rank);
  const size_t qt = (size_t)p->batch * p->num_q_heads * p->rank * 4;
  return rec + (qt + 255) / 256 * 256;
}

int check_append_params(const lrattn_append_params* p) {
  if (!p) return LRATTN_ERR_NULL;
  if (p->batch <= 0 || p->num_kv_heads <= 0 || p->model_dim <= 0 || p->rank <= 0 ||
      p->max_seq_len <= 0)
    return LRATTN_ERR_SHAPE;
  if ((p->x_dtype != LRATTN_BF16 && p->x_dtype != LRATTN_F16) || p->factor_dtype != p->x_dtype ||
      esize(p->latent_dtype) == 0)
    return LRATTN_ERR_DTYPE;
  if (checked_mul({p->batch, p->num_kv_heads, p->max_seq_len, p->rank, 4}) < 0)
    return LRATTN_ERR_SHAPE;
  if (!lrattn::append_supported(p->rank, p->batch, p->model_dim) || p->num_kv_heads > 65535)
    return LRATTN_ERR_UNSUPPORTED;
  return LRATTN_OK;
}

size_t append_ws_for(const lrattn_append_params* p) {
  return lrattn::append_workspace_bytes(p->num_kv_heads, p->batch, p->rank,
                                        lrattn::append_chunks(p->num_kv_heads, p->model_dim));
}
}  // namespace

int lrattn_append_workspace_size(const lrattn_append_params* p, size_t* bytes) {
  if (!bytes) return LRATTN_ERR_NULL;
  const int st = check_append_params(p);
  if (st != LRATTN_OK) return st;
  *bytes = append_ws_for(p);
  return LRATTN_OK;
}

int lrattn_append(const lrattn_append_params* p, const void* x, const void* A_K,
                  const void* A_V, const int32_t* positions, void* L_K, void* L_V,
                  float* scales, void* workspace, size_t workspace_bytes, lrattn_stream stream) {
  int st = check_append_params(p);
  if (st != LRATTN_OK) return st;
  if (!x || !A_K || !A_V || !positions || !L_K || !L_V) return LRATTN_ERR_NULL;
  if ((p->latent_dtype == LRATTN_I8) != (scales != nullptr)) return LRATTN_ERR_NULL;
  if (!aligned16(x) || !aligned16(A_K) || !aligned16(A_V) || !aligned16(positions) ||
      !aligned16(L_K) || !aligned16(L_V) || (scales && !aligned16(scales)))
    return LRATTN_ERR_ALIGN;
  if (!workspace) return LRATTN_ERR_WORKSPACE;
  if (!aligned16(workspace)) return LRATTN_ERR_ALIGN;
  if (workspace_bytes < append_ws_for(p)) return LRATTN_ERR_WORKSPACE;
  lrattn::AppendArgs a;
  a.x = x; a.AK = A_K; a.AV = A_V; a.positions = positions; a.LK = L_K; a.LV = L_V;
  a.scales = scales; a.ws = static_cast<float*>(workspace);
  a.B = p->batch; a.Hkv = p->num_kv_heads; a.D = p->model_dim; a.r = p->rank;
  a.T = p->max_seq_len; a.x_dtype = p->x_dtype; a.latent_dtype = p->latent_dtype;
  a.KS = lrattn::append_chunks(p->num_kv_heads, p->model_dim);
  if (lrattn::launch_append(a, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
    return LRATTN_ERR_HIP;
  return LRATTN_OK;
}

int lrattn_shared_workspace_size(const lrattn_params* p, size_t* bytes) {
  if (!bytes) return LRATTN_ERR_NULL;
  lrattn_params gp;
  Plan pl;
  const int st = check_shared(p, &gp, &pl);
  if (st != LRATTN_OK) return st;
  *bytes = shared_ws_bytes(p, pl);
  return LRATTN_OK;
}

int lrattn_shared_decode(const lrattn_params* p, const void* q, const void* L_K, const void* L_V,
                         const void* B_K, const void* B_V, const float* scales,
                         const int32_t* seq_lens, void* out, void* workspace,
                         size_t workspace_bytes, lrattn_stream stream) {
  lrattn_params gp;
  Plan pl;
  bool once = false;
  int st = check_shared(p, &gp, &pl, &once);
  if (st == LRATTN_OK) st = check_partition_ptrs(p, q, L_K, L_V, B_K, scales, seq_lens);
  if (st == LRATTN_OK) st = check_combine_ptrs(B_V, seq_lens, out);
  if (st == LRATTN_OK && !workspace) st = LRATTN_ERR_WORKSPACE;
  if (st == LRATTN_OK && !aligned16(workspace)) st = LRATTN_ERR_ALIGN;
  if (st == LRATTN_OK && workspace_bytes < shared_ws_bytes(p, pl)) st = LRATTN_ERR_WORKSPACE;
  if (st != LRATTN_OK) return st;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int G = shared_group(p);
  float* qt = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                       lrattn::records_bytes(p->batch, p->num_q_heads, pl.P,
                                                             p->rank));
  lrattn::AbsorbHeadsArgs ab;
  ab.q = q; ab.BK = B_K; ab.qt = qt;
  ab.B = p->batch; ab.Hq = p->num_q_heads; ab.d = p->head_dim; ab.r = p->rank;
  ab.hpf = 1;  // one factor block per query head
  ab.q_dtype = p->q_dtype; ab.f_dtype = p->factor_dtype; ab.qscale = qscale_for(p);
  if (lrattn::launch_absorb_heads(ab, s) != hipSuccess) return LRATTN_ERR_HIP;
  if (once) {
    lrattn::SharedOnceArgs oa;
    oa.qt = qt; oa.LK = L_K; oa.LV = L_V; oa.seq_lens = seq_lens;
    oa.ws = static_cast<float*>(workspace);
    oa.B = p->batch; oa.Hq = p->num_q_heads; oa.S = p->num_kv_heads; oa.T = p->max_seq_len;
    oa.P = pl.P; oa.Stok = pl.S;
    if (lrattn::launch_shared_once(p->rank, oa, s) != hipSuccess) return LRATTN_ERR_HIP;
    auto ca = combine_args(p, pl, B_V, seq_lens, out, workspace);
    ca.factor_per_head = 1;
    if (lrattn::launch_combine(G, ca, s) != hipSuccess) return LRATTN_ERR_HIP;
    return LRATTN_OK;
  }
  auto pa = partition_args(p, pl, q, L_K, L_V, B_K, scales, seq_lens, workspace);
  pa.qt_pre = qt;
  pa.HG = p->num_q_heads / G;                    // head groups
  pa.hps = p->num_q_heads / p->num_kv_heads;     // heads per latent stream
  // the head groups of a tile share its latents: keep them on one XCD
  pa.xcd_group = pa.HG > 1 && (int64_t)8 * pa.HG * ((pl.P * (int64_t)p->batch + 7) / 8) < (1LL << 31);
  if (lrattn::launch_partition(p->latent_dtype, p->rank, G, pa, s) != hipSuccess)
    return LRATTN_ERR_HIP;
  auto ca = combine_args(p, pl, B_V, seq_lens, out, workspace);
  ca.factor_per_head = 1;
  if (lrattn::launch_combine(G, ca, s) != hipSuccess) return LRATTN_ERR_HIP;
  return LRATTN_OK;
}

size_t lrattn_probe_sink_floats(void) { return (size_t)lrattn::kProbeBlocks; }

int lrattn_probe_read(const void* src, size_t bytes, float* sink, lrattn_stream stream) {
  if (!src || !sink) return LRATTN_ERR_NULL;
  if (bytes == 0 || bytes % 16) return LRATTN_ERR_SHAPE;
  if (!aligned16(src) || !aligned16(sink)) return LRATTN_ERR_ALIGN;
  if (lrattn::launch_probe_read(src, bytes, sink, reinterpret_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return LRATTN_ERR_HIP;
  return LRATTN_OK;
}

int lrattn_probe_copy(void* dst, const void* src, size_t bytes, lrattn_stream stream) {
  if (!src || !dst) return LRATTN_ERR_NULL;
  if (bytes == 0 || bytes % 16) return LRATTN_ERR_SHAPE;
  if (!aligned16(src) || !aligned16(dst)) return LRATTN_ERR_ALIGN;
  if (lrattn::launch_probe_copy(dst, src, bytes, reinterpret_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return LRATTN_ERR_HIP;
  return LRATTN_OK;
}

}  // extern "C"
