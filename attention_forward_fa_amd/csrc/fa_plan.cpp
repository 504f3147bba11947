// Phase 1 of the two-phase forward: argument validation and planning.
//
// Host-only and synchronous: reads tensor descriptors, never device memory.
// The checks follow the constraint lists of the aclnnFlashAttentionScore page
// (约束与限制) and the aclnnFlashAttentionVarLenScoreV5 page (约束说明 and the
// 返回值 error table); the status numbers are the pages' aclnn codes.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <stdlib.h>

#include <new>

#include "fa_fwd.h"
#include "fa_params.h"
#include "fa_merge.h"
#include "fa_plan.h"

namespace {

thread_local char g_err[512] = "no error";

fa_status fail(fa_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

enum Layout { L_BNSD, L_BSND, L_BSH, L_SBH, L_TND, L_BAD };

Layout parse_layout(const char* s) {
  if (!strcmp(s, "BNSD")) return L_BNSD;
  if (!strcmp(s, "BSND")) return L_BSND;
  if (!strcmp(s, "BSH")) return L_BSH;
  if (!strcmp(s, "SBH")) return L_SBH;
  if (!strcmp(s, "TND")) return L_TND;
  return L_BAD;
}

const char* dtype_name(int32_t dt) {
  switch (dt) {
    case FA_DTYPE_F32: return "f32";
    case FA_DTYPE_F16: return "f16";
    case FA_DTYPE_BF16: return "bf16";
    case FA_DTYPE_U8: return "u8";
    case FA_DTYPE_BOOL: return "bool";
    case FA_DTYPE_I32: return "i32";
    case FA_DTYPE_I64: return "i64";
  }
  return "?";
}

// A q/k/v-like tensor seen through its layout.
struct View {
  int64_t b, s, n, d;     // batch, rows, heads, head dim (TND: b = 1, s = T)
  int64_t sb, ss, sh;     // element strides
};

// Decode `t` in layout L.  For BSH/SBH the hidden size H is split by either a
// known head count (heads > 0) or a known head dim (hdim > 0).
fa_status decode(const fa_tensor* t, Layout L, const char* name, int64_t heads, int64_t hdim, View* v) {
  const int want = (L == L_BNSD || L == L_BSND) ? 4 : 3;
  if (t->ndim != want)
    return fail(FA_ERR_PARAM_INVALID, "%s: %d dims, layout needs %d", name, t->ndim, want);
  for (int i = 0; i < want; ++i)
    if (t->shape[i] < 0) return fail(FA_ERR_PARAM_INVALID, "%s: negative extent in dim %d", name, i);
  if (t->stride[want - 1] != 1 && t->shape[want - 1] > 1)
    return fail(FA_ERR_PARAM_INVALID, "%s: last dimension must be contiguous (stride 1)", name);
  switch (L) {
    case L_BNSD:
      *v = {t->shape[0], t->shape[2], t->shape[1], t->shape[3], t->stride[0], t->stride[2], t->stride[1]};
      return FA_OK;
    case L_BSND:
      *v = {t->shape[0], t->shape[1], t->shape[2], t->shape[3], t->stride[0], t->stride[1], t->stride[2]};
      return FA_OK;
    case L_TND:
      *v = {1, t->shape[0], t->shape[1], t->shape[2], 0, t->stride[0], t->stride[1]};
      return FA_OK;
    case L_BSH:
    case L_SBH: {
      const int64_t H = t->shape[2];
      int64_t n, d;
      if (heads > 0) {
        if (H % heads) return fail(FA_ERR_UNSUPPORTED, "%s: H=%lld not divisible by %lld heads", name, (long long)H, (long long)heads);
        n = heads;
        d = H / heads;
      } else {
        if (hdim <= 0 || H % hdim)
          return fail(FA_ERR_UNSUPPORTED, "%s: H=%lld not a multiple of head dim %lld", name, (long long)H, (long long)hdim);
        d = hdim;
        n = H / hdim;
      }
      if (L == L_BSH)
        *v = {t->shape[0], t->shape[1], n, d, t->stride[0], t->stride[1], d};
      else
        *v = {t->shape[1], t->shape[0], n, d, t->stride[1], t->stride[0], d};
      return FA_OK;
    }
    default:
      return fail(FA_ERR_PARAM_INVALID, "bad layout");
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool vec_ok(const void* p, const View& v) {
  // 16-byte vector access of 16-bit elements at every row start
  return aligned16(p) && (v.sb % 8 == 0) && (v.ss % 8 == 0) && (v.sh % 8 == 0);
}

// Window bounds are clamped to +-2^28, which is "unbounded" for sequences of
// at most 2^24 rows and keeps every row +- bound sum inside int32 on the device.
int64_t clamp_window(int64_t x) {
  const int64_t lim = (int64_t)1 << 28;
  return x < -lim ? -lim : (x > lim ? lim : x);
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

extern "C" const char* fa_last_error_message(void) { return g_err; }

void fa_set_error(const char* msg) { snprintf(g_err, sizeof(g_err), "%s", msg); }

extern "C" void fa_plan_destroy(fa_plan* plan) { delete plan; }

extern "C" int32_t fa_plan_describe(const fa_plan* plan, char* buf, size_t len) {
  if (!plan || !buf) return -1;
  const fa::Params& p = plan->p;
  const int n = snprintf(buf, len,
                         "kernel=%s dtype=%s d=%d dr=%d dv=%d bm=%d bn=%d grid=%d block=%d ws=%llu "
                         "varlen=%d band=%d pre=%d next=%d mask=%d sink=%d "
                         "nq=%d nkv=%d tiles_per_head=%d tile_search=%d reverse=%d pse=%d pse_lds=%d kv_splits=%d",
                         plan->kind == fa::KERNEL_MFMA_PP ? "mfma_pp" : (plan->kind == fa::KERNEL_MFMA ? "mfma" : "generic"),
                         dtype_name(plan->dtype), p.d, p.dr,
                         p.dv, plan->bm, plan->bn, p.num_wg, plan->block, (unsigned long long)plan->ws_bytes,
                         p.varlen, p.band, p.pre, p.next, p.has_mask, p.has_sink, p.nq, p.nkv,
                         p.tiles_per_head, p.tile_search, p.reverse_tiles, p.has_pse, p.pse_lds, p.kv_splits);
  return n;
}

extern "C" fa_status fa_fwd_get_workspace_size(
    const fa_tensor* query, const fa_tensor* query_rope, const fa_tensor* key, const fa_tensor* key_rope,
    const fa_tensor* value, const fa_tensor* real_shift, const fa_tensor* atten_mask, const fa_tensor* sink,
    const fa_tensor* cu_seqlens_q, const fa_tensor* cu_seqlens_kv, const int64_t* q_start_idx,
    const int64_t* kv_start_idx, double scale_value, double keep_prob,
    int64_t pre_tokens, int64_t next_tokens, int64_t head_num, const char* input_layout, int64_t inner_precise,
    int64_t sparse_mode, int32_t causal, const char* softmax_out_layout, const fa_tensor* softmax_max,
    const fa_tensor* softmax_sum, const fa_tensor* attention_out, uint64_t* workspace_size, fa_plan** plan) {
  if (plan) *plan = nullptr;
  // ---- required pointers (161001)
  if (!query) return fail(FA_ERR_PARAM_NULLPTR, "query is NULL");
  if (!key) return fail(FA_ERR_PARAM_NULLPTR, "key is NULL");
  if (!value) return fail(FA_ERR_PARAM_NULLPTR, "value is NULL");
  if (!attention_out) return fail(FA_ERR_PARAM_NULLPTR, "attention_out is NULL");
  if (!input_layout) return fail(FA_ERR_PARAM_NULLPTR, "input_layout is NULL");
  if (!workspace_size) return fail(FA_ERR_PARAM_NULLPTR, "workspace_size is NULL");
  if (!plan) return fail(FA_ERR_PARAM_NULLPTR, "plan is NULL");
  if ((query_rope == nullptr) != (key_rope == nullptr))
    return fail(FA_ERR_PARAM_NULLPTR, "query_rope and key_rope must be given together");

  // ---- dtypes and formats (161002)
  const Layout L = parse_layout(input_layout);
  if (L == L_BAD) return fail(FA_ERR_PARAM_INVALID, "input_layout '%s' not one of BNSD BSND BSH SBH TND", input_layout);
  const int32_t dt = query->dtype;
  if (dt != FA_DTYPE_F32 && dt != FA_DTYPE_F16 && dt != FA_DTYPE_BF16)
    return fail(FA_ERR_PARAM_INVALID, "query dtype %s not f32/f16/bf16", dtype_name(dt));
  if (key->dtype != dt || value->dtype != dt)
    return fail(FA_ERR_PARAM_INVALID, "query/key/value dtypes differ");
  if (attention_out->dtype != dt) return fail(FA_ERR_PARAM_INVALID, "attention_out dtype must equal query's");
  if (query_rope) {
    if (dt == FA_DTYPE_F32) return fail(FA_ERR_PARAM_INVALID, "rope parts need f16/bf16 inputs");
    if (query_rope->dtype != dt || key_rope->dtype != dt)
      return fail(FA_ERR_PARAM_INVALID, "rope dtypes must equal query's");
  }
  if (atten_mask && atten_mask->dtype != FA_DTYPE_U8 && atten_mask->dtype != FA_DTYPE_BOOL)
    return fail(FA_ERR_PARAM_INVALID, "atten_mask dtype %s not u8/bool", dtype_name(atten_mask->dtype));
  if (sink && sink->dtype != FA_DTYPE_F32) return fail(FA_ERR_PARAM_INVALID, "sink dtype must be f32");
  if (real_shift && real_shift->dtype != dt) return fail(FA_ERR_PARAM_INVALID, "real_shift dtype must equal query's");
  if (softmax_max && softmax_max->dtype != FA_DTYPE_F32) return fail(FA_ERR_PARAM_INVALID, "softmax_max must be f32");
  if (softmax_sum && softmax_sum->dtype != FA_DTYPE_F32) return fail(FA_ERR_PARAM_INVALID, "softmax_sum must be f32");
  const char* sol = softmax_out_layout ? softmax_out_layout : "";
  const bool stats_same_as_input = !strcmp(sol, "same_as_input");
  if (!stats_same_as_input && sol[0] != '\0')
    return fail(FA_ERR_PARAM_INVALID, "softmax_out_layout '%s' not \"\" or \"same_as_input\"", sol);
  if (L == L_TND) {
    if (!cu_seqlens_q || !cu_seqlens_kv) return fail(FA_ERR_PARAM_NULLPTR, "TND needs cu_seqlens_q and cu_seqlens_kv");
    if (cu_seqlens_q->dtype != FA_DTYPE_I32 || cu_seqlens_kv->dtype != FA_DTYPE_I32)
      return fail(FA_ERR_PARAM_INVALID, "cu_seqlens must be i32");
    if (cu_seqlens_q->ndim != 1 || cu_seqlens_kv->ndim != 1)
      return fail(FA_ERR_PARAM_INVALID, "cu_seqlens must be 1-D");
  }

  // ---- attributes (561103)
  if (real_shift && query_rope) return fail(FA_ERR_UNSUPPORTED, "real_shift cannot be combined with rope inputs");
  if (keep_prob != 1.0) return fail(FA_ERR_UNSUPPORTED, "keep_prob must be 1 (no dropout)");
  if (sparse_mode != 0) return fail(FA_ERR_UNSUPPORTED, "sparse_mode %lld unsupported (only 0)", (long long)sparse_mode);
  if (inner_precise < 0 || inner_precise > 2) return fail(FA_ERR_UNSUPPORTED, "inner_precise must be 0, 1 or 2");
  if (!isfinite(scale_value) || scale_value < 0.0) return fail(FA_ERR_UNSUPPORTED, "scale_value must be finite and >= 0");
  if (head_num <= 0 || head_num > 256) return fail(FA_ERR_UNSUPPORTED, "head_num %lld outside 1..256", (long long)head_num);
  if (L != L_TND && (cu_seqlens_q || cu_seqlens_kv))
    return fail(FA_ERR_UNSUPPORTED, "cu_seqlens only apply to TND");

  // ---- shapes
  fa_status st;
  View q, k, v, o, qr{}, kr{};
  if ((st = decode(query, L, "query", head_num, 0, &q))) return st;
  if (q.n != head_num) return fail(FA_ERR_UNSUPPORTED, "head_num %lld != query heads %lld", (long long)head_num, (long long)q.n);
  if ((st = decode(key, L, "key", 0, q.d, &k))) return st;
  if (L == L_BSH || L == L_SBH) {
    if ((st = decode(value, L, "value", k.n, 0, &v))) return st;
    if ((st = decode(attention_out, L, "attention_out", q.n, 0, &o))) return st;
  } else {
    if ((st = decode(value, L, "value", 0, 0, &v))) return st;
    if ((st = decode(attention_out, L, "attention_out", 0, 0, &o))) return st;
  }
  if (q.d != k.d) return fail(FA_ERR_UNSUPPORTED, "query D %lld != key D %lld", (long long)q.d, (long long)k.d);
  if (v.d > k.d) return fail(FA_ERR_UNSUPPORTED, "value D %lld > key D %lld", (long long)v.d, (long long)k.d);
  if (q.d < 1 || v.d < 1) return fail(FA_ERR_UNSUPPORTED, "head dim must be >= 1");
  if (k.n < 1 || q.n % k.n) return fail(FA_ERR_UNSUPPORTED, "Nq %lld not a multiple of Nkv %lld", (long long)q.n, (long long)k.n);
  if (v.n != k.n) return fail(FA_ERR_UNSUPPORTED, "value heads %lld != key heads %lld", (long long)v.n, (long long)k.n);
  if (L != L_TND && (q.b != k.b || q.b != v.b)) return fail(FA_ERR_UNSUPPORTED, "batch sizes of q/k/v differ");
  if (k.s != v.s) return fail(FA_ERR_UNSUPPORTED, "key rows %lld != value rows %lld", (long long)k.s, (long long)v.s);
  if (o.b != q.b || o.s != q.s || o.n != q.n || o.d != v.d)
    return fail(FA_ERR_UNSUPPORTED, "attention_out shape must be query's with last dim Dv");
  int64_t dr = 0;
  if (query_rope) {
    if ((st = decode(query_rope, L, "query_rope", q.n, 0, &qr))) return st;
    if ((st = decode(key_rope, L, "key_rope", k.n, 0, &kr))) return st;
    if (qr.b != q.b || qr.s != q.s || qr.n != q.n) return fail(FA_ERR_UNSUPPORTED, "query_rope shape must match query's");
    if (kr.b != k.b || kr.s != k.s || kr.n != k.n) return fail(FA_ERR_UNSUPPORTED, "key_rope shape must match key's");
    if (qr.d != kr.d || qr.d < 1) return fail(FA_ERR_UNSUPPORTED, "rope head dims differ");
    dr = qr.d;
  }
  if (q.d + dr > 256 || v.d > 256)
    return fail(FA_ERR_UNSUPPORTED, "head dim D+Dr=%lld or Dv=%lld above 256", (long long)(q.d + dr), (long long)v.d);
  if (q.s > (1 << 24) || k.s > (1 << 24)) return fail(FA_ERR_UNSUPPORTED, "more than 2^24 rows");

  int64_t nbatch = q.b;
  if (L == L_TND) {
    nbatch = cu_seqlens_q->shape[0] - 1;
    if (nbatch < 1 || cu_seqlens_kv->shape[0] != cu_seqlens_q->shape[0])
      return fail(FA_ERR_UNSUPPORTED, "cu_seqlens need B+1 >= 2 entries, equal for q and kv");
    if (nbatch > 20000) return fail(FA_ERR_UNSUPPORTED, "more than 20000 sequences");
    if (!cu_seqlens_q->data || !cu_seqlens_kv->data) return fail(FA_ERR_PARAM_NULLPTR, "cu_seqlens data is NULL");
  }

  if (real_shift) {
    const fa_tensor* r = real_shift;
    if (!r->data) return fail(FA_ERR_PARAM_NULLPTR, "real_shift data is NULL");
    if (L == L_TND) {
      if (r->ndim != 1) return fail(FA_ERR_UNSUPPORTED, "TND real_shift must be 1-D: [N*Sq_i*Skv_i over sequences]");
      if (r->stride[0] != 1) return fail(FA_ERR_PARAM_INVALID, "real_shift must be contiguous");
    } else {
      if (r->ndim != 4 || !(r->shape[0] == q.b || r->shape[0] == 1) || r->shape[1] != q.n || r->shape[3] != k.s)
        return fail(FA_ERR_UNSUPPORTED, "real_shift shape must be [B|1, N, Sq, Skv]");
      if (r->shape[2] != q.s)
        return fail(FA_ERR_UNSUPPORTED, "real_shift must have Sq rows (the compressed last-1024-rows form is not supported)");
      if (r->stride[3] != 1) return fail(FA_ERR_PARAM_INVALID, "real_shift last dimension must be contiguous");
    }
  }

  if (atten_mask) {
    const fa_tensor* m = atten_mask;
    if (L == L_TND) {
      if (m->ndim != 2) return fail(FA_ERR_UNSUPPORTED, "TND takes a 2-D atten_mask");
    } else if (m->ndim == 4) {
      if (!((m->shape[0] == q.b || m->shape[0] == 1) && (m->shape[1] == q.n || m->shape[1] == 1) &&
            m->shape[2] == q.s && m->shape[3] == k.s))
        return fail(FA_ERR_UNSUPPORTED, "atten_mask shape must be [B|1, N|1, Sq, Skv]");
      if (m->shape[1] == 1 && m->shape[0] != 1 && m->shape[0] != q.b)
        return fail(FA_ERR_UNSUPPORTED, "atten_mask shape must be [B|1, N|1, Sq, Skv]");
    } else if (m->ndim == 2) {
      if (m->shape[0] != q.s || m->shape[1] != k.s) return fail(FA_ERR_UNSUPPORTED, "atten_mask shape must be [Sq, Skv]");
    } else {
      return fail(FA_ERR_UNSUPPORTED, "atten_mask must be 2-D or 4-D");
    }
    if (!m->data && m->shape[0] * m->shape[1] > 0) return fail(FA_ERR_PARAM_NULLPTR, "atten_mask data is NULL");
  }
  if (sink) {
    if (sink->ndim != 1 || sink->shape[0] != q.n) return fail(FA_ERR_UNSUPPORTED, "sink must be [Nq]");
    if (!sink->data) return fail(FA_ERR_PARAM_NULLPTR, "sink data is NULL");
  }
  const fa_tensor* stats[2] = {softmax_max, softmax_sum};
  int64_t st_sb = 0, st_ss = 0, st_sh = 0;
  for (int i = 0; i < 2; ++i) {
    const fa_tensor* s = stats[i];
    if (!s) continue;
    const char* nm = i ? "softmax_sum" : "softmax_max";
    int64_t sb, ss, sh;
    if (L == L_TND) {
      if (s->ndim != 3 || s->shape[2] != 8) return fail(FA_ERR_UNSUPPORTED, "%s must be [N,T,8] or [T,N,8]", nm);
      if (stats_same_as_input) {
        if (s->shape[0] != q.s || s->shape[1] != q.n) return fail(FA_ERR_UNSUPPORTED, "%s must be [T,N,8]", nm);
        sb = 0; ss = s->stride[0]; sh = s->stride[1];
      } else {
        if (s->shape[0] != q.n || s->shape[1] != q.s) return fail(FA_ERR_UNSUPPORTED, "%s must be [N,T,8]", nm);
        sb = 0; sh = s->stride[0]; ss = s->stride[1];
      }
    } else {
      if (s->ndim != 4 || s->shape[0] != q.b || s->shape[1] != q.n || s->shape[2] != q.s || s->shape[3] != 8)
        return fail(FA_ERR_UNSUPPORTED, "%s must be [B,N,Sq,8]", nm);
      sb = s->stride[0]; sh = s->stride[1]; ss = s->stride[2];
    }
    if (s->stride[s->ndim - 1] != 1) return fail(FA_ERR_PARAM_INVALID, "%s: last dimension must be contiguous", nm);
    if (i == 0) {
      st_sb = sb; st_ss = ss; st_sh = sh;
    } else if (softmax_max && (sb != st_sb || ss != st_ss || sh != st_sh)) {
      return fail(FA_ERR_UNSUPPORTED, "softmax_max and softmax_sum must have equal strides");
    } else {
      st_sb = sb; st_ss = ss; st_sh = sh;
    }
  }

  // ---- window
  const bool band = atten_mask != nullptr || causal != 0;
  int64_t pre = clamp_window(pre_tokens), nxt = clamp_window(next_tokens);
  if (causal && nxt > 0) nxt = 0;
  if (band && pre + nxt < 0)
    return fail(FA_ERR_UNSUPPORTED, "preTokens + nextTokens < 0: the window is empty");
  // Outer split: the chunk's rows start at q_start and its keys at kv_start
  // in the whole sequence, and the window is a condition on global positions:
  // -pre <= (j + kv_start) - (i + q_start) <= next, i.e. the same test on
  // local positions with both bounds moved by q_start - kv_start.
  const int64_t qs = q_start_idx ? *q_start_idx : 0, ks = kv_start_idx ? *kv_start_idx : 0;
  if (qs < 0 || ks < 0 || qs > ((int64_t)1 << 26) || ks > ((int64_t)1 << 26))
    return fail(FA_ERR_UNSUPPORTED, "q_start_idx / kv_start_idx must be in [0, 2^26]");
  pre = clamp_window(pre - (qs - ks));
  nxt = clamp_window(nxt + (qs - ks));

  // ---- kernel choice
  fa_plan* pl = new (std::nothrow) fa_plan();
  if (!pl) return fail(FA_ERR_UNSUPPORTED, "out of host memory");
  fa::Params& p = pl->p;
  pl->dtype = dt;
  const bool stats_vec = (!softmax_max || aligned16(softmax_max->data)) && (!softmax_sum || aligned16(softmax_sum->data)) &&
                         st_sb % 4 == 0 && st_ss % 4 == 0 && st_sh % 4 == 0;
  // Dqk = Dv + 64 without rope inputs or pse: on the matrix cores the last 64
  // dims of q and k serve as the rope part (the same rows and strides), so the
  // kernels see D = Dv and Dr = 64.
  const bool tail_split = !query_rope && !real_shift && (dt == FA_DTYPE_F16 || dt == FA_DTYPE_BF16) &&
                          q.d == v.d + 64 && (v.d == 64 || v.d == 96 || v.d == 128);
  const int64_t dmain = tail_split ? v.d : q.d;
  const int64_t drm = tail_split ? 64 : dr;
  // The four-wave kernel stages a key block with 32-bit byte offsets from
  // the block's first row: row r < 64 of K, V (and Krope) at r * row bytes
  // must stay below 2^31 (a strided view or an SBH layout can have rows far
  // apart).
  const int64_t esz_in = dt == FA_DTYPE_F32 ? 4 : 2;
  int64_t max_row_b = (k.ss > v.ss ? k.ss : v.ss) * esz_in;
  if (query_rope && kr.ss * esz_in > max_row_b) max_row_b = kr.ss * esz_in;
  const bool block_offsets_fit = (int64_t)fa::kMfmaBN * max_row_b < ((int64_t)1 << 31);
  // (D, Dr, Dv) the four-wave kernel is built for: Dv == D in {64, 96, 128}
  // with 0 or 64 rope dims; without rope, D = 256 with Dv = 256, and D in
  // {96, 128, 256} with a smaller Dv in {64, 96, 128} (the head dims of the
  // FAS page's constraints, with the V5 page's kD >= vD)
  auto dv_ok = [](int64_t d) { return d == 64 || d == 96 || d == 128; };
  const bool dims_mfma = ((dmain == 64 || dmain == 96 || dmain == 128) && v.d == dmain && (drm == 0 || drm == 64)) ||
                         (dmain == 256 && drm == 0 && v.d == 256) ||
                         ((dmain == 96 || dmain == 128 || dmain == 256) && drm == 0 && dv_ok(v.d) && v.d < dmain);
  const bool mfma_shape = (dt == FA_DTYPE_F16 || dt == FA_DTYPE_BF16) && dims_mfma && vec_ok(query->data, q) &&
                          vec_ok(key->data, k) &&
                          vec_ok(value->data, v) && vec_ok(attention_out->data, o) &&
                          (!query_rope || (vec_ok(query_rope->data, qr) && vec_ok(key_rope->data, kr))) && stats_vec;
  const bool mfma_ok = mfma_shape && block_offsets_fit;
  // Family: the two-group (ping-pong) matrix-core kernel for long dense
  // sequences at D = 128 without rope whose window cuts at most the causal
  // side or is at least 2048 keys wide (narrower windows waste a larger share
  // of the steps, since the two groups' key ranges differ by 128 rows), with
  // at least one workgroup per compute unit (it measures faster there: one
  // K / V stream serves 256 query rows); the four-wave
  // matrix-core kernel wherever else it applies (short or varlen sequences,
  // rope, sliding windows, D = 64, grids too small for the two-group kernel,
  // which it may split along the keys); the generic kernel for everything
  // else.  FA_FWD_KERNEL=mfma|pp|generic forces a family (tests and
  // benchmarks); forcing a matrix-core family on a shape it does not cover is
  // an error.
  // the two-group kernel addresses a sequence's K / V rows with 32-bit byte
  // offsets from its first row, up to Skv + 4 blocks of rows
  const int64_t esz = dt == FA_DTYPE_F32 ? 4 : 2;
  int64_t row_b = k.ss > v.ss ? k.ss : v.ss;
  if (query_rope && kr.ss > row_b) row_b = kr.ss;
  const bool pp_fits = (k.s + 4 * fa::kMfmaBN) * row_b * esz < ((int64_t)1 << 31);
  const bool pp_pref = pp_fits && dmain == 128 && drm == 0 && L != L_TND && q.s >= 1024 && k.s >= 1024 &&
                       (!band || pre >= k.s - 1 || pre + nxt >= 2047) && !real_shift &&
                       q.b * q.n * cdiv(q.s, fa::kMfmaPpBM) >= fa::kNumCUs;
  int kind = mfma_ok ? (pp_pref ? fa::KERNEL_MFMA_PP : fa::KERNEL_MFMA) : fa::KERNEL_GENERIC;
  if (const char* force = getenv("FA_FWD_KERNEL")) {
    if (!strcmp(force, "generic")) {
      kind = fa::KERNEL_GENERIC;
    } else if (!strcmp(force, "mfma") || !strcmp(force, "pp")) {
      if (mfma_shape && !block_offsets_fit) {
        delete pl;
        return fail(FA_ERR_UNSUPPORTED, "FA_FWD_KERNEL=%s: 64 key rows span 2 GiB or more (32-bit block offsets)",
                    force);
      }
      if (!mfma_ok) {
        delete pl;
        return fail(FA_ERR_UNSUPPORTED, "FA_FWD_KERNEL=%s: shape, dtype or alignment not covered", force);
      }
      if (!strcmp(force, "pp") && real_shift) {
        delete pl;
        return fail(FA_ERR_UNSUPPORTED, "FA_FWD_KERNEL=pp: the two-group kernel takes no real_shift");
      }
      if (!strcmp(force, "pp") && !((dmain == 64 || dmain == 128) && v.d == dmain)) {
        delete pl;
        return fail(FA_ERR_UNSUPPORTED, "FA_FWD_KERNEL=pp: the two-group kernel has D = Dv = 64 or 128 only");
      }
      if (!strcmp(force, "pp") && !pp_fits) {
        delete pl;
        return fail(FA_ERR_UNSUPPORTED, "FA_FWD_KERNEL=pp: K / V rows of one sequence span 2 GiB or more");
      }
      kind = !strcmp(force, "pp") ? fa::KERNEL_MFMA_PP : fa::KERNEL_MFMA;
    } else if (force[0] != '\0') {
      delete pl;
      return fail(FA_ERR_UNSUPPORTED, "FA_FWD_KERNEL='%s' not one of pp, mfma, generic", force);
    }
  }
  pl->kind = kind;
  pl->bm = kind == fa::KERNEL_MFMA_PP ? fa::kMfmaPpBM : (kind == fa::KERNEL_MFMA ? fa::kMfmaBM : fa::kGenericBM);
  pl->bn = kind == fa::KERNEL_GENERIC ? fa::kGenericBN : fa::kMfmaBN;
  pl->block = kind == fa::KERNEL_MFMA_PP ? fa::kMfmaPpThreads
                                         : (kind == fa::KERNEL_MFMA ? fa::kMfmaThreads : fa::kGenericThreads);

  p.q = query->data; p.k = key->data; p.v = value->data;
  p.qr = query_rope ? query_rope->data : nullptr;
  p.kr = key_rope ? key_rope->data : nullptr;
  const bool tail_rope = tail_split && kind != fa::KERNEL_GENERIC;  // the generic kernel takes Dv < D as it is
  if (tail_rope) {
    const int64_t esz = dt == FA_DTYPE_F32 ? 4 : 2;
    p.qr = static_cast<const char*>(query->data) + v.d * esz;
    p.kr = static_cast<const char*>(key->data) + v.d * esz;
    qr = q;
    kr = k;
  }
  p.o = attention_out->data;
  p.smax = softmax_max ? static_cast<float*>(softmax_max->data) : nullptr;
  p.ssum = softmax_sum ? static_cast<float*>(softmax_sum->data) : nullptr;
  p.mask = atten_mask ? static_cast<const uint8_t*>(atten_mask->data) : nullptr;
  p.sink = sink ? static_cast<const float*>(sink->data) : nullptr;
  p.cu_q = L == L_TND ? static_cast<const int32_t*>(cu_seqlens_q->data) : nullptr;
  p.cu_kv = L == L_TND ? static_cast<const int32_t*>(cu_seqlens_kv->data) : nullptr;
  p.tile_prefix = nullptr;  // set from the workspace in phase 2
  p.tile_map = nullptr;
  p.q_sb = q.sb; p.q_ss = q.ss; p.q_sh = q.sh;
  p.k_sb = k.sb; p.k_ss = k.ss; p.k_sh = k.sh;
  p.v_sb = v.sb; p.v_ss = v.ss; p.v_sh = v.sh;
  p.qr_sb = qr.sb; p.qr_ss = qr.ss; p.qr_sh = qr.sh;
  p.kr_sb = kr.sb; p.kr_ss = kr.ss; p.kr_sh = kr.sh;
  p.o_sb = o.sb; p.o_ss = o.ss; p.o_sh = o.sh;
  p.st_sb = st_sb; p.st_ss = st_ss; p.st_sh = st_sh;
  p.m_sb = p.m_sh = p.m_sq = p.m_sk = 0;
  p.m_rows = p.m_cols = 0;
  if (atten_mask) {
    const fa_tensor* m = atten_mask;
    if (m->ndim == 4) {
      p.m_sb = m->shape[0] > 1 ? m->stride[0] : 0;
      p.m_sh = m->shape[1] > 1 ? m->stride[1] : 0;
      p.m_sq = m->stride[2];
      p.m_sk = m->stride[3];
    } else {
      p.m_sq = m->stride[0];
      p.m_sk = m->stride[1];
      p.m_rows = (int32_t)(m->shape[0] < (1 << 24) ? m->shape[0] : (1 << 24));
      p.m_cols = (int32_t)(m->shape[1] < (1 << 24) ? m->shape[1] : (1 << 24));
    }
  }
  p.pse = real_shift ? real_shift->data : nullptr;
  p.pse_off = nullptr;  // set from the workspace in phase 2
  p.has_pse = real_shift != nullptr;
  p.ps_sb = p.ps_sh = p.ps_sq = 0;
  p.pse_len = 0;
  if (real_shift) {
    const fa_tensor* r = real_shift;
    p.pse_len = 1;
    for (int i = 0; i < r->ndim; ++i) p.pse_len *= r->shape[i];
    if (r->ndim == 4) {
      p.ps_sb = r->shape[0] > 1 ? r->stride[0] : 0;
      p.ps_sh = r->stride[1];
      p.ps_sq = r->stride[2];
      // every element the strides can reach bounds the reads
      p.pse_len = (r->shape[0] - 1) * p.ps_sb + (r->shape[1] - 1) * p.ps_sh + (r->shape[2] - 1) * p.ps_sq + r->shape[3];
    }
  }
  p.nbatch = (int32_t)nbatch;
  p.nq = (int32_t)q.n;
  p.nkv = (int32_t)k.n;
  p.group = (int32_t)(q.n / k.n);
  p.varlen = L == L_TND;
  p.sq = p.varlen ? 0 : (int32_t)q.s;
  p.skv = p.varlen ? 0 : (int32_t)k.s;
  p.tq = p.varlen ? (int32_t)q.s : 0;
  p.tkv = p.varlen ? (int32_t)k.s : 0;
  p.d = (int32_t)(tail_rope ? dmain : q.d);
  p.dr = (int32_t)(tail_rope ? drm : dr);
  p.dv = (int32_t)v.d;
  p.scale = (float)scale_value;
  // The kernels turn excluded scores into -inf and rely on -inf * c = -inf;
  // a zero scale is replaced by a positive one far below any score's
  // resolution (every weight is then exactly 1, as with scale 0).
  p.scale_log2 = (float)(scale_value * 1.4426950408889634);
  if (!(p.scale_log2 > 1e-30f)) p.scale_log2 = 1e-30f;
  // pse enters the raw (unscaled) score accumulator as pse * inv_scale, so
  // that times scale_log2 it becomes pse * log2(e)
  p.inv_scale = (float)(1.4426950408889634 / (double)p.scale_log2);
  p.band = band;
  p.pre = (int32_t)pre;
  p.next = (int32_t)nxt;
  p.has_mask = atten_mask != nullptr;
  p.has_sink = sink != nullptr;
  const int64_t max_keys = k.s;  // per-sequence lengths are at most this
  p.mask_vec4 = p.has_mask && !p.varlen && p.m_sk == 1 && (reinterpret_cast<uintptr_t>(p.mask) & 3u) == 0 &&
                p.m_sq % 4 == 0 && p.m_sb % 4 == 0 && p.m_sh % 4 == 0;
  p.reverse_tiles = band && nxt < max_keys - 1;
  p.pse_vec4 = p.has_pse && !p.varlen && (reinterpret_cast<uintptr_t>(p.pse) & 7u) == 0 && p.ps_sq % 4 == 0 &&
               p.ps_sb % 4 == 0 && p.ps_sh % 4 == 0;
  // pse through LDS reads the 128 x 64 tile with 32-bit byte offsets from
  // its first element: row r < 128 at r * row bytes must stay below 2^31
  p.pse_lds = p.has_pse && !p.varlen && dr == 0 && (reinterpret_cast<uintptr_t>(p.pse) & 15u) == 0 &&
              p.ps_sq % 8 == 0 && p.ps_sb % 8 == 0 && p.ps_sh % 8 == 0 &&
              (int64_t)fa::kMfmaBM * p.ps_sq * esz_in < ((int64_t)1 << 31);

  const int64_t bm = pl->bm;
  int64_t tiles, wg;
  // Workspace: [tile prefix, int32] [tile map, 8 x int32 per tile] (TND with
  // more than kTileSearchMaxSeqs sequences) [pse block offsets, int64, TND
  // with pse] [mask block classes, u8, with a mask], each part 16-byte aligned.
  uint64_t ws = 0;
  pl->ws_map_off = pl->ws_pse_off = pl->ws_cls_off = 0;
  p.tile_search = 0;
  p.tile_bm = (int32_t)bm;
  if (p.varlen) {
    tiles = cdiv(q.s, bm) + nbatch;
    wg = q.s > 0 ? tiles * q.n : 0;
    p.tile_search = nbatch <= fa::kTileSearchMaxSeqs;
    if (!p.tile_search) {
      ws = (uint64_t)(nbatch + 1) * sizeof(int32_t);
      pl->ws_map_off = (ws + 15) / 16 * 16;
      ws = pl->ws_map_off + (uint64_t)tiles * 8 * sizeof(int32_t);
    }
    if (p.has_pse) {
      pl->ws_pse_off = (ws + 15) / 16 * 16;
      ws = pl->ws_pse_off + (uint64_t)(nbatch + 1) * sizeof(int64_t);
    }
  } else {
    tiles = cdiv(q.s, bm);
    wg = tiles * q.b * q.n;
  }
  // Key split (dense, 4-wave kernel): a grid that leaves workgroup slots of
  // the chip empty gets up to kMaxKvSplits workgroups per query tile, each
  // over kv_splits-th of the keys (whole key blocks, at least kMinSplitBlocks
  // of them), and a merge pass.  FA_FWD_KV_SPLIT=n forces n ranges (1 = off;
  // tests and benchmarks).
  p.kv_splits = 1;
  p.split_keys = 0;
  p.part_o = p.part_ml = nullptr;
  pl->ws_part_off = 0;
  if (kind == fa::KERNEL_MFMA && !p.varlen && wg > 0 && k.s > 0) {
    // workgroup slots of the chip: two per CU while the kernel's LDS (two
    // K / V stages of 64 rows of Dqk + Dv elements, and the 16 KiB pse tile
    // when pse goes through LDS) fits in 80 KiB, else one
    const int64_t lds_b = 2 * (int64_t)fa::kMfmaBN * (dmain + drm + v.d) * esz_in + (p.pse_lds ? 16 * 1024 : 0);
    const int64_t slots = lds_b <= 80 * 1024 ? fa::kWgSlots : fa::kNumCUs;
    int64_t want = slots / wg;
    if (want > fa::kMaxKvSplits) want = fa::kMaxKvSplits;
    const int64_t max_by_len = k.s / ((int64_t)fa::kMinSplitBlocks * pl->bn);
    if (want > max_by_len) want = max_by_len;
    // Not with pse: its [Sq, Skv] bias per head dominates the HBM bytes, and
    // the fp32 partials would add a fifth to them (B1 N8 S4096: 68 MB on 304)
    // for a few percent of speed.
    if (real_shift) want = 1;
    if (const char* force = getenv("FA_FWD_KV_SPLIT")) {
      char* end = nullptr;
      const long n = strtol(force, &end, 10);
      if (force[0] != '\0') {
        if (*end != '\0' || n < 1 || n > fa::kMaxKvSplits) {
          delete pl;
          return fail(FA_ERR_UNSUPPORTED, "FA_FWD_KV_SPLIT='%s' not a count in 1..%d", force, fa::kMaxKvSplits);
        }
        want = n;
      }
    }
    if (want >= 2) {
      const int64_t keys = cdiv(cdiv(k.s, want), pl->bn) * pl->bn;
      p.kv_splits = (int32_t)cdiv(k.s, keys);
      p.split_keys = (int32_t)keys;
      wg *= p.kv_splits;
    }
  }
  p.mask_cls = nullptr;
  p.cls_nh = p.cls_tiles = p.cls_kblocks = p.cls_slices = 0;
  if (p.has_mask) {
    // dense: one class table per (mask batch, mask head) slice over [Sq, Skv];
    // TND: one table over the 2-D mask [m_rows, m_cols]
    const fa_tensor* m = atten_mask;
    int64_t nslices = 1, rows = q.s, cols = k.s;
    if (p.varlen) {
      rows = m->shape[0];
      cols = m->shape[1];
    } else if (m->ndim == 4) {
      nslices = m->shape[0] * m->shape[1];
      p.cls_nh = (int32_t)m->shape[1];
    }
    if (p.cls_nh == 0) p.cls_nh = 1;
    if (nslices >= ((int64_t)1 << 31)) {
      delete pl;
      return fail(FA_ERR_UNSUPPORTED, "mask with %lld slices too large", (long long)nslices);
    }
    p.cls_slices = (int32_t)nslices;
    p.cls_tiles = (int32_t)cdiv(rows, fa::kClsRows);
    p.cls_kblocks = (int32_t)cdiv(cols, fa::kClsKeys);
    pl->ws_cls_off = (ws + 15) / 16 * 16;
    // padded to 16 bytes: the kernels read the table a dword at a time
    ws = pl->ws_cls_off + ((uint64_t)nslices * p.cls_tiles * p.cls_kblocks + 15) / 16 * 16;
  }
  if (p.kv_splits > 1) {
    // fp32 partial outputs [kv_splits][rows][dv], then {max, sum} [kv_splits][rows][2]
    const uint64_t rows = (uint64_t)p.kv_splits * q.b * q.n * q.s;
    pl->ws_part_off = (ws + 15) / 16 * 16;
    ws = pl->ws_part_off + rows * (uint64_t)(v.d + 2) * sizeof(float);
  }
  pl->ws_bytes = ws;
  if (wg >= ((int64_t)1 << 31)) {
    delete pl;
    return fail(FA_ERR_UNSUPPORTED, "grid of %lld workgroups too large", (long long)wg);
  }
  p.tiles_per_head = (int32_t)tiles;
  p.num_wg = (int32_t)wg;
  *workspace_size = pl->ws_bytes;
  *plan = pl;
  // FA_LOG (set and not "0"): one line per plan on stderr with the kernel,
  // tile, grid and workspace phase 1 chose
  if (const char* log = getenv("FA_LOG")) {
    if (log[0] != '\0' && strcmp(log, "0") != 0) {
      char buf[512];
      fa_plan_describe(pl, buf, sizeof(buf));
      fprintf(stderr, "[fa_fwd] plan %s layout=%s\n", buf, input_layout);
    }
  }
  return FA_OK;
}

// ---------------------------------------------------------------------------
// Merge of partial results (outer split along the keys)
// ---------------------------------------------------------------------------

namespace {

// Strides (batch, head, row) of an [..., 8] statistics tensor for layout L.
fa_status stats_view(const fa_tensor* s, Layout L, bool same_as_input, const View& o, const char* nm, int64_t* sb,
                     int64_t* sh, int64_t* ss) {
  if (s->dtype != FA_DTYPE_F32) return fail(FA_ERR_PARAM_INVALID, "%s must be f32", nm);
  if (L == L_TND) {
    if (s->ndim != 3 || s->shape[2] != 8) return fail(FA_ERR_UNSUPPORTED, "%s must be [N,T,8] or [T,N,8]", nm);
    if (same_as_input) {
      if (s->shape[0] != o.s || s->shape[1] != o.n) return fail(FA_ERR_UNSUPPORTED, "%s must be [T,N,8]", nm);
      *sb = 0; *ss = s->stride[0]; *sh = s->stride[1];
    } else {
      if (s->shape[0] != o.n || s->shape[1] != o.s) return fail(FA_ERR_UNSUPPORTED, "%s must be [N,T,8]", nm);
      *sb = 0; *sh = s->stride[0]; *ss = s->stride[1];
    }
  } else {
    if (s->ndim != 4 || s->shape[0] != o.b || s->shape[1] != o.n || s->shape[2] != o.s || s->shape[3] != 8)
      return fail(FA_ERR_UNSUPPORTED, "%s must be [B,N,Sq,8]", nm);
    *sb = s->stride[0]; *sh = s->stride[1]; *ss = s->stride[2];
  }
  if (s->stride[s->ndim - 1] != 1) return fail(FA_ERR_PARAM_INVALID, "%s: last dimension must be contiguous", nm);
  if (!s->data) return fail(FA_ERR_PARAM_NULLPTR, "%s data is NULL", nm);
  return FA_OK;
}

}  // namespace

extern "C" fa_status fa_fwd_merge(int32_t n_parts, const fa_tensor* part_out, const fa_tensor* part_max,
                                  const fa_tensor* part_sum, const char* input_layout, int64_t head_num,
                                  const char* softmax_out_layout, const fa_tensor* attention_out,
                                  const fa_tensor* softmax_max, const fa_tensor* softmax_sum, void* stream) {
  if (!part_out || !part_max || !part_sum) return fail(FA_ERR_PARAM_NULLPTR, "part arrays are NULL");
  if (!attention_out || !input_layout) return fail(FA_ERR_PARAM_NULLPTR, "attention_out / input_layout is NULL");
  if (n_parts < 1 || n_parts > fa::kMergeMaxParts)
    return fail(FA_ERR_UNSUPPORTED, "n_parts %d outside 1..%d", n_parts, fa::kMergeMaxParts);
  const Layout L = parse_layout(input_layout);
  if (L == L_BAD) return fail(FA_ERR_PARAM_INVALID, "input_layout '%s' not one of BNSD BSND BSH SBH TND", input_layout);
  const char* sol = softmax_out_layout ? softmax_out_layout : "";
  const bool same = !strcmp(sol, "same_as_input");
  if (!same && sol[0] != '\0') return fail(FA_ERR_PARAM_INVALID, "softmax_out_layout '%s' invalid", sol);
  const int32_t dt = attention_out->dtype;
  if (dt != FA_DTYPE_F32 && dt != FA_DTYPE_F16 && dt != FA_DTYPE_BF16)
    return fail(FA_ERR_PARAM_INVALID, "attention_out dtype %s not f32/f16/bf16", dtype_name(dt));
  if (head_num <= 0 || head_num > 256) return fail(FA_ERR_UNSUPPORTED, "head_num outside 1..256");
  fa_status st;
  View o;
  if ((st = decode(attention_out, L, "attention_out", head_num, 0, &o))) return st;
  if (o.d > 256 || o.n != head_num) return fail(FA_ERR_UNSUPPORTED, "attention_out heads / dim out of range");
  if (!attention_out->data) return fail(FA_ERR_PARAM_NULLPTR, "attention_out data is NULL");
  fa::MergeParams mp{};
  mp.nparts = n_parts;
  mp.dv = (int32_t)o.d;
  mp.nbatch = (int32_t)o.b;
  mp.nheads = (int32_t)o.n;
  mp.nrows = (int32_t)o.s;
  mp.o = attention_out->data;
  mp.o_sb = o.sb; mp.o_ss = o.ss; mp.o_sh = o.sh;
  for (int c = 0; c < n_parts; ++c) {
    View pv;
    if (part_out[c].dtype != dt) return fail(FA_ERR_PARAM_INVALID, "part %d output dtype differs", c);
    if ((st = decode(&part_out[c], L, "part output", head_num, 0, &pv))) return st;
    if (pv.b != o.b || pv.s != o.s || pv.n != o.n || pv.d != o.d)
      return fail(FA_ERR_UNSUPPORTED, "part %d output shape differs from attention_out", c);
    if (!part_out[c].data) return fail(FA_ERR_PARAM_NULLPTR, "part %d output data is NULL", c);
    mp.po[c] = part_out[c].data;
    mp.po_sb[c] = pv.sb; mp.po_ss[c] = pv.ss; mp.po_sh[c] = pv.sh;
    int64_t sb, sh, ss, sb2, sh2, ss2;
    if ((st = stats_view(&part_max[c], L, same, o, "part softmax_max", &sb, &sh, &ss))) return st;
    if ((st = stats_view(&part_sum[c], L, same, o, "part softmax_sum", &sb2, &sh2, &ss2))) return st;
    if (sb != sb2 || sh != sh2 || ss != ss2) return fail(FA_ERR_UNSUPPORTED, "part %d stats strides differ", c);
    mp.pm[c] = static_cast<const float*>(part_max[c].data);
    mp.pl[c] = static_cast<const float*>(part_sum[c].data);
    mp.pst_sb[c] = sb; mp.pst_sh[c] = sh; mp.pst_ss[c] = ss;
  }
  mp.st_sb = mp.st_sh = mp.st_ss = 0;
  if (softmax_max || softmax_sum) {
    int64_t sb = 0, sh = 0, ss = 0, sb2 = 0, sh2 = 0, ss2 = 0;
    if (softmax_max && (st = stats_view(softmax_max, L, same, o, "softmax_max", &sb, &sh, &ss))) return st;
    if (softmax_sum && (st = stats_view(softmax_sum, L, same, o, "softmax_sum", &sb2, &sh2, &ss2))) return st;
    if (softmax_max && softmax_sum && (sb != sb2 || sh != sh2 || ss != ss2))
      return fail(FA_ERR_UNSUPPORTED, "softmax_max and softmax_sum must have equal strides");
    if (!softmax_max) { sb = sb2; sh = sh2; ss = ss2; }
    mp.st_sb = sb; mp.st_sh = sh; mp.st_ss = ss;
  }
  mp.m = softmax_max ? static_cast<float*>(softmax_max->data) : nullptr;
  mp.l = softmax_sum ? static_cast<float*>(softmax_sum->data) : nullptr;
  const int e = fa::merge_launch(mp, dt, stream);
  if (e != 0) {
    fail(FA_ERR_RUNTIME, "merge kernel launch failed (HIP error %d)", e);
    return FA_ERR_RUNTIME;
  }
  return FA_OK;
}
