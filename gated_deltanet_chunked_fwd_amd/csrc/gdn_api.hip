// C ABI of libgdn: argument validation, workspace carving and the launch
// sequence.  Declarations and the full contract are in include/gdn.h.
#include <climits>
#include <cmath>
#include <cstring>

#include "gdn.h"
#include "gdn_launch.h"

namespace {

using gdn::kChunk;

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Records the caller's timing events around one stage (no-op without events).
struct StageMark {
  hipEvent_t* ev;
  hipStream_t s;
  int stage;
  StageMark(const gdn_opts* o, int stage_, hipStream_t s_)
      : ev(o ? o->stage_events : nullptr), s(s_), stage(stage_) {
    if (ev) (void)hipEventRecord(ev[2 * stage], s);
  }
  ~StageMark() {
    if (ev) (void)hipEventRecord(ev[2 * stage + 1], s);
  }
};

int validate_shape(const gdn_shape* s) {
  if (!s) return GDN_ERR_ARG;
  if (s->B < 1 || s->T < 0 || s->H < 1 || s->N < 0) return GDN_ERR_ARG;
  if (s->T > INT_MAX / 2 || s->H > 65535) return GDN_ERR_ARG;
  if ((s->dk != 64 && s->dk != 128) || (s->dv != 64 && s->dv != 128)) return GDN_ERR_UNSUPPORTED;
  if ((s->qkv_dtype != GDN_BF16 && s->qkv_dtype != GDN_F32) ||
      (s->beta_dtype != GDN_BF16 && s->beta_dtype != GDN_F32))
    return GDN_ERR_UNSUPPORTED;
  if (s->cu_seqlens_host) {
    if (s->B != 1 || s->N < 1) return GDN_ERR_ARG;
    const int32_t* cu = s->cu_seqlens_host;
    if (cu[0] != 0 || cu[s->N] != s->T) return GDN_ERR_ARG;
    for (int64_t n = 0; n < s->N; ++n)
      if (cu[n + 1] < cu[n]) return GDN_ERR_ARG;
  } else if (s->N != s->B) {
    return GDN_ERR_ARG;
  }
  return GDN_OK;
}

int64_t total_chunks(const gdn_shape* s) {
  if (!s->cu_seqlens_host) return s->B * ((s->T + kChunk - 1) / kChunk);
  int64_t c = 0;
  for (int64_t n = 0; n < s->N; ++n)
    c += (s->cu_seqlens_host[n + 1] - s->cu_seqlens_host[n] + kChunk - 1) / kChunk;
  return c;
}

struct Layout {
  size_t tmat = 0, chunk_off = 0, total = 0;
};

Layout layout(const gdn_shape* s) {
  Layout L;
  const size_t esz = s->qkv_dtype == GDN_BF16 ? 2 : 4;
  size_t off = 0;
  L.tmat = off;
  off += align_up((size_t)total_chunks(s) * (size_t)s->H * kChunk * kChunk * esz);
  L.chunk_off = off;
  off += align_up((size_t)(s->N + 1) * sizeof(int32_t));
  L.total = off;
  return L;
}

gdn::Problem make_problem(const void* q, const void* k, const void* v, const float* g,
                          const void* beta, const float* h0, const int32_t* cu, float scale,
                          void* o, float* hT, const gdn_shape* s) {
  gdn::Problem p;
  p.q = q; p.k = k; p.v = v; p.g = g; p.beta = beta; p.h0 = h0; p.cu = cu;
  p.chunk_off = nullptr; p.o = o; p.hT = hT;
  p.T = s->T;
  p.total_chunks = total_chunks(s);
  p.N = (int)s->N; p.H = (int)s->H; p.dk = (int)s->dk; p.dv = (int)s->dv;
  p.qkv_bf16 = s->qkv_dtype == GDN_BF16;
  p.beta_bf16 = s->beta_dtype == GDN_BF16;
  p.scale = scale;
  return p;
}

int check_inputs(const void* k, const float* g, const void* beta, const int32_t* cu,
                 const gdn_shape* s) {
  if ((cu == nullptr) != (s->cu_seqlens_host == nullptr)) return GDN_ERR_ARG;
  if (s->T > 0 && (!k || !g || !beta)) return GDN_ERR_ARG;
  if (k && !aligned(k, 16)) return GDN_ERR_ARG;
  if (g && !aligned(g, 4)) return GDN_ERR_ARG;
  if (beta && !aligned(beta, s->beta_dtype == GDN_BF16 ? 2 : 4)) return GDN_ERR_ARG;
  if (cu && !aligned(cu, 4)) return GDN_ERR_ARG;
  return GDN_OK;
}

}  // namespace

extern "C" {

int64_t gdn_total_chunks(const gdn_shape* shape) {
  int rc = validate_shape(shape);
  if (rc != GDN_OK) return rc;
  return total_chunks(shape);
}

int gdn_chunk_fwd_workspace_bytes(const gdn_shape* shape, const gdn_opts* opts, size_t* bytes) {
  (void)opts;
  int rc = validate_shape(shape);
  if (rc != GDN_OK) return rc;
  if (!bytes) return GDN_ERR_ARG;
  *bytes = layout(shape).total;
  return GDN_OK;
}

int gdn_chunk_fwd(const void* q, const void* k, const void* v, const float* g, const void* beta,
                  const float* initial_state, const int32_t* cu_seqlens, float scale, void* o,
                  float* final_state, const gdn_shape* shape, const gdn_opts* opts,
                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int rc = validate_shape(shape);
  if (rc != GDN_OK) return rc;
  rc = check_inputs(k, g, beta, cu_seqlens, shape);
  if (rc != GDN_OK) return rc;
  if (shape->T > 0 && (!q || !v || !o)) return GDN_ERR_ARG;
  if ((q && !aligned(q, 16)) || (v && !aligned(v, 16)) || (o && !aligned(o, 16)) ||
      (initial_state && !aligned(initial_state, 16)) || (final_state && !aligned(final_state, 16)))
    return GDN_ERR_ARG;
  if (!std::isfinite(scale)) return GDN_ERR_ARG;
  if (opts && opts->value_block != 0 && opts->value_block != 64 && opts->value_block != 128)
    return GDN_ERR_ARG;
  const Layout L = layout(shape);
  if (workspace_bytes < L.total || (L.total > 0 && !workspace) || !aligned(workspace, kAlign))
    return GDN_ERR_WORKSPACE;

  char* ws = static_cast<char*>(workspace);
  gdn::Problem p = make_problem(q, k, v, g, beta, initial_state, cu_seqlens, scale, o,
                                final_state, shape);
  if (cu_seqlens) {
    p.chunk_off = reinterpret_cast<int32_t*>(ws + L.chunk_off);
    if (gdn::launch_chunk_offsets(cu_seqlens, p.N, const_cast<int32_t*>(p.chunk_off), stream) !=
        hipSuccess)
      return GDN_ERR_HIP;
  }
  void* tmat = ws + L.tmat;
  {
    StageMark mark(opts, GDN_STAGE_INVERSE, stream);
    if (gdn::launch_chunk_inverse(p, tmat, stream) != hipSuccess) return GDN_ERR_HIP;
  }

  gdn::FwdPlan plan;
  plan.Tmat = tmat;
  plan.seg_chunks = INT_MAX / 2;
  plan.seg_off = nullptr;
  plan.units = (int64_t)p.N * p.H;
  plan.value_block = opts ? opts->value_block : 0;
  {
    StageMark mark(opts, GDN_STAGE_FORWARD, stream);
    if (gdn::launch_fused_forward(p, plan, stream) != hipSuccess) return GDN_ERR_HIP;
  }
  return GDN_OK;
}

int gdn_chunk_inverse(const void* k, const float* g, const void* beta, const int32_t* cu_seqlens,
                      const gdn_shape* shape, void* t_out, void* workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  int rc = validate_shape(shape);
  if (rc != GDN_OK) return rc;
  rc = check_inputs(k, g, beta, cu_seqlens, shape);
  if (rc != GDN_OK) return rc;
  const int64_t nch = total_chunks(shape);
  if (nch > 0 && (!t_out || !aligned(t_out, 16))) return GDN_ERR_ARG;
  gdn::Problem p = make_problem(nullptr, k, nullptr, g, beta, nullptr, cu_seqlens, 1.f, nullptr,
                                nullptr, shape);
  if (cu_seqlens) {
    const size_t need = align_up((size_t)(shape->N + 1) * sizeof(int32_t));
    if (!workspace || workspace_bytes < need || !aligned(workspace, kAlign)) return GDN_ERR_WORKSPACE;
    p.chunk_off = static_cast<int32_t*>(workspace);
    if (gdn::launch_chunk_offsets(cu_seqlens, p.N, static_cast<int32_t*>(workspace), stream) !=
        hipSuccess)
      return GDN_ERR_HIP;
  }
  if (gdn::launch_chunk_inverse(p, t_out, stream) != hipSuccess) return GDN_ERR_HIP;
  return GDN_OK;
}

const char* gdn_status_str(int status) {
  switch (status) {
    case GDN_OK: return "ok";
    case GDN_ERR_ARG: return "invalid argument";
    case GDN_ERR_UNSUPPORTED: return "unsupported configuration";
    case GDN_ERR_WORKSPACE: return "workspace missing or too small";
    case GDN_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"
