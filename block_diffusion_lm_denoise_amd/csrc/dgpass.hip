// dgpass.hip -- the C ABI of libdgpass: validation, workspace carving and the
// launch sequence of a prefill and of a denoising pass.  See include/dgpass.h.
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "launch.h"

using namespace dg;

namespace {

constexpr uint32_t MODEL_MAGIC = 0x44475041u;  // "DGPA"

size_t al(size_t x) { return (x + 255) & ~(size_t)255; }
int esize(int dt) { return dt == DG_F32 ? 4 : dt == DG_BF16 ? 2 : 1; }
// bytes of n elements of storage type dt (MXFP4: two codes per byte)
size_t nbytes(size_t n, int dt) { return dt == DG_MXFP4 ? n / 2 : n * esize(dt); }

constexpr int MIN_TILE = 32;      // smallest expert row tile (sizes the tile list)
constexpr int STREAM_MAX_ROWS = 1024;  // dense projections: weight streaming up to this many rows
constexpr int ROUTE_MIN_ROWS = 2048;   // fused routing kernel from this many token rows

struct Layout {
  size_t cov;       // [L][E] int32 expert counts of the last pass (offset 0)
  size_t x, u, qkv, o, x1, u2, rl, ids, gates, counts, offsets, perm, inv, tiles, ntiles, H, Y;
  size_t lpm, lpi, lps;
  size_t fixed;     // bytes before the attention split partials
  size_t po, pml, total;
  long part_cap;    // (row, head) entries of split partials the workspace holds
  int max_tiles;
};

// router logits: R x E floats, times the contraction splits of the router
// GEMM when few rows leave the GPU idle (partials summed by the top-k kernel)
constexpr size_t ROUTER_SPLIT_CAP = (size_t)1 << 21;   // floats of partials at most
int router_split(const dg_config& c, int rows) {
  const int nch = c.D * esize(c.act_dtype) / 128;   // packed pieces per router row
  const size_t re = (size_t)rows * c.E;
  int S = 1;
  // aim at >= 256 blocks: (E/64 column chunks) x (rows/32 row tiles) x S
  const long base = (long)((c.E + 63) / 64) * ((rows + 31) / 32);
  while (S < ROUTER_MAX_SPLIT && base * S < 256 && nch % (2 * S) == 0 && nch / (2 * S) >= 4 &&
         re * 2 * S <= ROUTER_SPLIT_CAP)
    S *= 2;
  return S;
}
size_t router_floats(const dg_config& c, int rows) {
  return (size_t)rows * c.E * router_split(c, rows);
}

// bytes of one (row, head) entry of the attention split partials: O in the
// activation type, then (m, l) in fp32
size_t part_entry_bytes(const dg_config& c) { return (size_t)c.hd * esize(c.act_dtype) + 2 * 4; }

// Workspace carve for `rows` token rows with room for `part_entries` (row,
// head) entries of attention split partials, which come last so that a
// call can use whatever room the caller's workspace leaves for them.
Layout layout(const dg_config& c, int rows, long part_entries) {
  Layout L{};
  const size_t a = esize(c.act_dtype);
  const size_t R = rows > 0 ? rows : 1;
  const size_t QKV = (size_t)(c.Hq + 2 * c.Hkv) * c.hd, QD = (size_t)c.Hq * c.hd;
  const size_t slots = R * c.k;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += al(bytes);
    return o;
  };
  L.cov = take((size_t)c.L * c.E * 4);
  L.x = take(R * c.D * a);
  L.u = take(R * c.D * a);
  L.qkv = take(R * QKV * a);
  L.o = take(R * QD * a);
  L.x1 = take(R * c.D * a);
  L.u2 = take(R * c.D * a);
  L.rl = take(router_floats(c, (int)R) * 4);
  L.ids = take(slots * 4);
  L.gates = take(slots * 4);
  L.counts = take((size_t)c.E * 4);
  L.offsets = take((size_t)(c.E + 1) * 4);
  L.perm = take(slots * 4);
  L.inv = take(slots * 4);
  L.max_tiles = (int)((slots + MIN_TILE - 1) / MIN_TILE) + c.E;
  L.tiles = take((size_t)L.max_tiles * 16);
  L.ntiles = take(4);
  L.H = take(slots * c.F * a);
  L.Y = take(slots * c.D * a);
  const size_t nt = (c.V + 63) / 64;  // LM-head partials per row (64-column chunks)
  L.lpm = take(R * nt * 4);
  L.lpi = take(R * nt * 4);
  L.lps = take(R * nt * 4);
  L.fixed = off;
  L.part_cap = part_entries > 0 ? part_entries : 0;
  L.po = take((size_t)L.part_cap * c.hd * a);   // partial O in the activation type
  L.pml = take((size_t)L.part_cap * 2 * 4);
  L.total = off;
  return L;
}

// the carve a call uses: the split partials it would like (its key counts),
// cut to what the caller's workspace holds beyond the fixed part
Layout call_layout(const dg_config& c, int rows, int max_keys, size_t ws_bytes) {
  Layout L = layout(c, rows, 0);
  const long want = attn_partial_entries(rows, c.Hq, max_keys);
  const size_t room = ws_bytes > L.fixed ? ws_bytes - L.fixed : 0;
  // the most entries whose two buffers (each rounded up to 256 bytes) fit the
  // room: a workspace sized by dg_workspace_bytes for these keys holds `want`
  auto need = [&](long n) { return al((size_t)n * c.hd * esize(c.act_dtype)) + al((size_t)n * 2 * 4); };
  long fit = (long)(room / part_entry_bytes(c));
  while (fit > 0 && need(fit) > room) fit--;
  return layout(c, rows, want < fit ? want : fit);
}

bool valid_cfg(const dg_config* c) {
  if (!c) return false;
  if (c->L < 1 || c->L > DG_MAX_LAYERS || c->D < 1 || c->Hq < 1 || c->Hkv < 1 || c->E < 1 ||
      c->k < 1 || c->F < 1 || c->V < 1 || !(c->eps >= 0.f))
    return false;
  return true;
}

dg_status supported_cfg(const dg_config* c) {
  if (c->D % 128 || c->F % 64) return DG_ERR_UNSUPPORTED;
  if (c->expert_dtype == DG_FP8E4M3 && c->F % 128) return DG_ERR_UNSUPPORTED;   // packed fp8 rows
  if (c->expert_dtype == DG_MXFP4 && (c->F % 256 || c->D % 256)) return DG_ERR_UNSUPPORTED;
  if (c->hd != 64 && c->hd != 128) return DG_ERR_UNSUPPORTED;
  if (c->Hq % c->Hkv) return DG_ERR_UNSUPPORTED;
  const int G = c->Hq / c->Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return DG_ERR_UNSUPPORTED;
  if ((c->Hq * c->hd) % 64) return DG_ERR_UNSUPPORTED;
  if (c->k > 8 || c->k > c->E || c->E > 256) return DG_ERR_UNSUPPORTED;
  if (c->act_dtype == DG_F32) {
    if (c->expert_dtype != DG_F32) return DG_ERR_UNSUPPORTED;
  } else if (c->act_dtype == DG_BF16) {
    if (c->expert_dtype != DG_BF16 && c->expert_dtype != DG_FP8E4M3 && c->expert_dtype != DG_MXFP4)
      return DG_ERR_UNSUPPORTED;
  } else {
    return DG_ERR_UNSUPPORTED;
  }
  return DG_OK;
}

bool model_ok(const dg_model* m) { return m && m->magic == MODEL_MAGIC; }

// everything after the attention of one layer: Wo + residual, norm, router,
// top-k, permutation, experts, combine + the next norm
struct Ctx {
  const dg_model* m;
  char* ws;
  Layout L;
  int R;          // token rows
  const dg_taps* taps;
  hipStream_t s;
  bool pass;      // denoising pass (writes coverage counts)
  int32_t* zero0 = nullptr;   // [nzero] counters the pass's last kernel adds to,
  int32_t* zero1 = nullptr;   // cleared by the last layer's combine
  int nzero = 0;
};

template <typename T>
T* at(const Ctx& c, size_t off) {
  return reinterpret_cast<T*>(c.ws + off);
}

void tap_copy(void* dst, const void* src, size_t bytes, hipStream_t s) {
  if (dst && bytes) (void)hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, s);
}

// record stage event [l][stage][which] of the caller's stage_events, if any
void stage_event(const dg_taps* t, int l, int stage, int which, hipStream_t s) {
  if (!t || !t->stage_events) return;
  void* e = t->stage_events[((size_t)l * DG_NSTAGES + stage) * 2 + which];
  if (e) (void)hipEventRecord((hipEvent_t)e, s);
}

// layer l's input rows replaced by the caller's (x and its first RMSNorm)
void inject_layer_input(const Ctx& c, int l) {
  const dg_taps* t = c.taps;
  if (!t || !t->inject_x) return;
  const dg_config& cf = c.m->cfg;
  const size_t a = esize(cf.act_dtype), bytes = (size_t)c.R * cf.D * a;
  (void)hipMemcpyAsync(at<void>(c, c.L.x), (const char*)t->inject_x + (size_t)l * bytes, bytes,
                       hipMemcpyDeviceToDevice, c.s);
  launch_rmsnorm(cf.act_dtype == DG_BF16 ? ACT_BF16 : ACT_F32, at<void>(c, c.L.x),
                 c.m->w.layers[l].g1, c.R, cf.D, cf.eps, at<void>(c, c.L.u), c.s);
}

// waves splitting the contraction: 4, or 2 when 4 would leave each wave an odd
// number of pieces (128 bytes of each weight row; the pipeline works on pairs)
int stream_kw(int K, int wdt) {
  // pieces of the contraction (MXFP4: half pieces of 128 elements)
  const int nch = wdt == DG_MXFP4 ? K / 128 : (int)(nbytes(K, wdt) / 128), per4 = (nch + 3) / 4;
  // MXFP4: 2 waves per contraction unless 4 get equal shares (the 768-wide
  // down projection: 43.8 against 47.9 us)
  if (wdt == DG_MXFP4) return (nch % 4 != 0 && nch % 2 == 0) ? 2 : 4;
  return (per4 % 2 == 1 && nch % 2 == 0) ? 2 : 4;
}

// dense projection C = A W^T (W rows stacked from up to three matrices):
// weight streaming for few rows, LDS-tiled MFMA GEMM for many
void dense_gemm(const Ctx& c, int mode, const void* A, int M, int K, const void* B0, int n1,
                const void* B1, int n2, const void* B2, int N, void* C, int ldc, const void* R,
                const CacheDst* cache) {
  const dg_config& cf = c.m->cfg;
  const int act = cf.act_dtype == DG_BF16 ? ACT_BF16 : ACT_F32;
  if (M <= STREAM_MAX_ROWS) {
    StreamGemm g{};
    g.A = A;
    g.M = M;
    g.K = K;
    g.W0 = B0;
    g.W1 = B1;
    g.W2 = B2;
    g.n1 = n1;
    g.n2 = n2;
    g.N = N;
    const int kw = stream_kw(K, cf.act_dtype);
    g.nchunks = (N + 64 * (4 / kw) - 1) / (64 * (4 / kw));
    g.out = C;
    g.ldo = ldc;
    g.R = R;
    if (cache) g.cache = *cache;
    const int sm = mode == GEMM_STORE ? SG_STORE : mode == GEMM_RESID ? SG_RESID
                 : mode == GEMM_F32 ? SG_F32 : SG_QKV_CACHE;
    launch_stream_gemm(act, cf.act_dtype, sm, kw, g, 0, c.s);
  } else {
    launch_gemm(act, mode, A, M, K, B0, n1, B1, n2, B2, N, C, ldc, R, cache, c.s);
  }
}

void moe_block(const Ctx& c, int l, const float* gnext) {
  const dg_config& cf = c.m->cfg;
  const dg_layer_weights& w = c.m->w.layers[l];
  const int act = cf.act_dtype == DG_BF16 ? ACT_BF16 : ACT_F32;
  const size_t a = esize(cf.act_dtype);
  const size_t R = c.R, D = cf.D, QD = (size_t)cf.Hq * cf.hd, E = cf.E, k = cf.k;
  const dg_taps* t = c.taps;
  hipStream_t s = c.s;

  // x1 = x + o Wo^T
  dense_gemm(c, GEMM_RESID, at<void>(c, c.L.o), c.R, (int)QD, w.wo, cf.D, nullptr, 0, nullptr, cf.D,
             at<void>(c, c.L.x1), cf.D, at<void>(c, c.L.x), nullptr);
  if (t) tap_copy(t->x1 ? (char*)t->x1 + l * R * D * a : nullptr, at<void>(c, c.L.x1), R * D * a, s);
  // RMSNorm + router logits (fp32) + top-k
  const float* rl = at<float>(c, c.L.rl);
  if (t && t->inject_router) rl = t->inject_router + (size_t)l * R * E;
  RouteArgs ra{at<void>(c, c.L.x1), w.g2, w.wr, c.R, cf.D, cf.E, cf.k, cf.eps,
               (t && t->inject_router) ? rl : nullptr, at<void>(c, c.L.u2),
               (t && t->router && !t->inject_router) ? at<float>(c, c.L.rl) : nullptr,
               at<int32_t>(c, c.L.ids), at<float>(c, c.L.gates)};
  // fused RMSNorm + router + top-k on 16-token tiles (bf16): only with many
  // tiles, since each tile is a serial chain (with few, the unfused kernels
  // spread the work over more of the chip)
  if (c.R <= STREAM_MAX_ROWS) {
    // the RMSNorm rides on the router and top-k launches (one dependent launch
    // fewer): the streamed router multiplies x1 by g2 in flight, and top-k
    // takes the row's rsqrt, scales the summed logits by it and writes u2
    const bool inj = t && t->inject_router;
    int S = 1;
    if (!inj) {
      // weight streaming with contraction splits; top-k sums the partials
      S = router_split(cf, c.R);
      StreamGemm g{};
      g.A = at<void>(c, c.L.x1);
      g.M = c.R;
      g.K = cf.D;
      g.W0 = w.wr;
      g.n1 = cf.E;
      g.N = cf.E;
      g.nchunks = (cf.E + 63) / 64;
      g.ksplit = S;
      g.gs = w.g2;
      g.out = at<void>(c, c.L.rl);
      g.ldo = cf.E;
      launch_stream_gemm(act, cf.act_dtype, SG_F32, 4, g, 0, s);
    }
    TopkNorm tn{at<void>(c, c.L.x1), w.g2, cf.D, cf.eps, at<void>(c, c.L.u2), inj ? 0 : 1};
    launch_topk_norm(act, const_cast<float*>(rl), S, c.R, cf.E, cf.k, at<int32_t>(c, c.L.ids),
                     at<float>(c, c.L.gates), tn, s);
  } else if (c.R < ROUTE_MIN_ROWS || !launch_route(act, ra, s)) {
    launch_rmsnorm(act, at<void>(c, c.L.x1), w.g2, c.R, cf.D, cf.eps, at<void>(c, c.L.u2), s);
    if (!(t && t->inject_router))
      dense_gemm(c, GEMM_F32, at<void>(c, c.L.u2), c.R, cf.D, w.wr, cf.E, nullptr, 0, nullptr, cf.E,
                 at<void>(c, c.L.rl), cf.E, nullptr, nullptr);
    launch_topk(const_cast<float*>(rl), 1, c.R, cf.E, cf.k, at<int32_t>(c, c.L.ids),
                at<float>(c, c.L.gates), s);
  }
  if (t) {
    tap_copy(t->u2 ? (char*)t->u2 + l * R * D * a : nullptr, at<void>(c, c.L.u2), R * D * a, s);
    tap_copy(t->router ? t->router + l * R * E : nullptr, rl, R * E * 4, s);
    tap_copy(t->ids ? t->ids + l * R * k : nullptr, at<void>(c, c.L.ids), R * k * 4, s);
    tap_copy(t->gates ? t->gates + l * R * k : nullptr, at<void>(c, c.L.gates), R * k * 4, s);
  }

  // permutation and row tiles
  const int avg = (int)(R * k / E);
  // weight streaming for few rows per expert; MXFP4 experts always stream
  // (the LDS-tiled grouped GEMMs take bf16 and fp8 weights)
  const bool stream = avg <= 64 || cf.expert_dtype == DG_MXFP4;
  const int tile_rows = stream ? stream_tile_rows(act, cf.expert_dtype) : group_tile_rows(act);
  const int max_tiles = (int)((R * k + tile_rows - 1) / tile_rows) + (int)E;
  int32_t* counts = c.pass ? at<int32_t>(c, c.L.cov) + l * E : at<int32_t>(c, c.L.counts);
  launch_plan(at<int32_t>(c, c.L.ids), c.R, cf.k, cf.E, tile_rows, counts, at<int32_t>(c, c.L.offsets),
              at<int32_t>(c, c.L.perm), at<int32_t>(c, c.L.inv), at<int4>(c, c.L.tiles),
              at<int32_t>(c, c.L.ntiles), s);
  if (t) {
    tap_copy(t->counts ? t->counts + l * E : nullptr, counts, E * 4, s);
    tap_copy(t->offsets ? t->offsets + l * (E + 1) : nullptr, at<void>(c, c.L.offsets), (E + 1) * 4, s);
    tap_copy(t->perm ? t->perm + l * R * k : nullptr, at<void>(c, c.L.perm), R * k * 4, s);
  }

  // experts over the union of the selected ones
  MoeW mw{w.wg, w.wu, w.wd, w.escale, cf.expert_dtype};
  StreamGemm g{};
  g.perm = at<int32_t>(c, c.L.perm);
  g.k = cf.k;
  g.escale = w.escale;
  g.S0 = w.wg_mx;
  g.S1 = w.wu_mx;
  g.tiles = at<int4>(c, c.L.tiles);
  g.ntiles = at<int32_t>(c, c.L.ntiles);
  stage_event(t, l, DG_STAGE_GATEUP, 0, s);
  if (stream) {
    g.A = at<void>(c, c.L.u2);
    g.K = cf.D;
    g.W0 = w.wg;
    g.W1 = w.wu;
    g.NW = cf.F;
    const int kw = stream_kw(cf.D, cf.expert_dtype);
    g.nchunks = cf.F / (32 * (4 / kw));
    g.out = at<void>(c, c.L.H);
    g.ldo = cf.F;
    launch_stream_gemm(act, cf.expert_dtype, SG_GATEUP, kw, g, max_tiles, s);
  } else {
    launch_gateup_lds(act, at<void>(c, c.L.u2), at<int32_t>(c, c.L.perm), cf.k, mw,
                      at<int4>(c, c.L.tiles), at<int32_t>(c, c.L.ntiles), max_tiles, cf.D, cf.F,
                      at<void>(c, c.L.H), s);
  }
  stage_event(t, l, DG_STAGE_GATEUP, 1, s);
  if (t && t->hmid)
    launch_unpermute(act, at<void>(c, c.L.H), at<int32_t>(c, c.L.inv), (int)(R * k), cf.F,
                     (char*)t->hmid + l * R * k * cf.F * a, s);
  stage_event(t, l, DG_STAGE_DOWN, 0, s);
  if (stream) {
    g.A = at<void>(c, c.L.H);
    g.K = cf.F;
    g.W0 = w.wd;
    g.W1 = nullptr;
    g.S0 = w.wd_mx;
    g.S1 = nullptr;
    g.NW = cf.D;
    g.N = cf.D;
    const int kw = stream_kw(cf.F, cf.expert_dtype);
    g.nchunks = cf.D / (64 * (4 / kw));
    g.out = at<void>(c, c.L.Y);
    g.ldo = cf.D;
    launch_stream_gemm(act, cf.expert_dtype, SG_DOWN, kw, g, max_tiles, s);
  } else {
    launch_down_lds(act, at<void>(c, c.L.H), mw, at<int4>(c, c.L.tiles), at<int32_t>(c, c.L.ntiles),
                    max_tiles, cf.D, cf.F, at<void>(c, c.L.Y), s);
  }
  stage_event(t, l, DG_STAGE_DOWN, 1, s);
  if (t && t->yexp)
    launch_unpermute(act, at<void>(c, c.L.Y), at<int32_t>(c, c.L.inv), (int)(R * k), cf.D,
                     (char*)t->yexp + l * R * k * D * a, s);

  // x = x1 + sum_j g_j y_j; u = next norm
  launch_combine_norm(act, at<void>(c, c.L.x1), at<void>(c, c.L.Y), at<float>(c, c.L.gates),
                      at<int32_t>(c, c.L.inv), c.R, cf.k, cf.D, gnext, cf.eps, at<void>(c, c.L.x),
                      at<void>(c, c.L.u), s, l + 1 == cf.L ? c.zero0 : nullptr,
                      l + 1 == cf.L ? c.zero1 : nullptr, c.nzero);
  if (t) tap_copy(t->xout ? (char*)t->xout + l * R * D * a : nullptr, at<void>(c, c.L.x), R * D * a, s);
}

dg_status check_hip() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? DG_OK : DG_ERR_HIP;
}

// Workspace of the allocation-free pass: a file-scope device array (each GPU
// the library runs on holds its own copy until the process ends).  Host code
// never passes the array's name to a kernel: it is a host-side stand-in, not
// a device address.  The device address is looked up once per device with
// that device current, and that pointer is what the kernels receive.
static __device__ __align__(256) char scratch[DG_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES];

// the current device's copy of `scratch`, or null with *st set
void* scratch_for_current_device(dg_status* st) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) {
    *st = DG_ERR_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      *st = DG_ERR_HIP;
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *st = DG_OK;
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* dg_status_str(dg_status s) {
  switch (s) {
    case DG_OK: return "ok";
    case DG_ERR_INVALID: return "invalid argument";
    case DG_ERR_CAPACITY: return "KV cache capacity exceeded";
    case DG_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case DG_ERR_WORKSPACE: return "workspace too small";
    case DG_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

dg_status dg_model_init(dg_model* m, const dg_config* cfg, const dg_weights* w) {
  if (!m || !valid_cfg(cfg) || !w) return DG_ERR_INVALID;
  dg_status st = supported_cfg(cfg);
  if (st != DG_OK) return st;
  if (!w->emb || !w->gf || !w->lm) return DG_ERR_INVALID;
  for (int l = 0; l < cfg->L; l++) {
    const dg_layer_weights& x = w->layers[l];
    if (!x.g1 || !x.wq || !x.wk || !x.wv || !x.wo || !x.g2 || !x.wr || !x.wg || !x.wu || !x.wd)
      return DG_ERR_INVALID;
    if ((cfg->expert_dtype == DG_FP8E4M3) != (x.escale != nullptr)) return DG_ERR_INVALID;
    const bool mx = cfg->expert_dtype == DG_MXFP4;
    if (mx != (x.wg_mx != nullptr) || mx != (x.wu_mx != nullptr) || mx != (x.wd_mx != nullptr))
      return DG_ERR_INVALID;
  }
  memset(m, 0, sizeof(*m));
  m->cfg = *cfg;
  m->w = *w;
  m->magic = MODEL_MAGIC;
  return DG_OK;
}

size_t dg_workspace_bytes(const dg_config* cfg, int32_t max_rows, int32_t max_keys) {
  if (!valid_cfg(cfg) || max_rows < 1 || max_keys < 0) return 0;
  return layout(*cfg, max_rows, attn_partial_entries(max_rows, cfg->Hq, max_keys)).total;
}

// causal prefill of T tokens per request; with argmax/conf set (a decoding
// step) the last layer runs in full and the LM head reads its output
static dg_status prefill(const dg_model* m, dg_kv* kv, const int32_t* tokens, int32_t B, int32_t T,
                         const dg_taps* taps, void* ws, size_t ws_bytes, void* stream,
                         int32_t* argmax, float* conf) {
  const bool head = argmax != nullptr;
  if (!model_ok(m) || !kv || !kv->len || !tokens || !ws) return DG_ERR_INVALID;
  if (head && !conf) return DG_ERR_INVALID;
  if (B < 1 || B > DG_MAX_BATCH || T < 1 || kv->cap < 1) return DG_ERR_INVALID;
  const dg_config& cf = m->cfg;
  for (int l = 0; l < cf.L; l++)
    if (!kv->k[l] || !kv->v[l]) return DG_ERR_INVALID;
  Lens lens{};
  int maxkeys = 0;
  for (int b = 0; b < B; b++) {
    if (kv->len[b] < 0 || kv->len[b] > kv->cap) return DG_ERR_INVALID;
    if ((long)kv->len[b] + T > kv->cap) return DG_ERR_CAPACITY;
    lens.v[b] = kv->len[b];
    maxkeys = kv->len[b] + T > maxkeys ? kv->len[b] + T : maxkeys;
  }
  if ((long)B * T > (1L << 20)) return DG_ERR_UNSUPPORTED;
  const int R = B * T;
  Ctx c{m, (char*)ws, call_layout(cf, R, maxkeys, ws_bytes), R, taps, (hipStream_t)stream, false};
  if (c.L.total > ws_bytes) return DG_ERR_WORKSPACE;

  (void)hipGetLastError();  // clear a stale error so the status below is ours
  const int act = cf.act_dtype == DG_BF16 ? ACT_BF16 : ACT_F32;
  const size_t a = esize(cf.act_dtype);
  const int QD = cf.Hq * cf.hd, KD = cf.Hkv * cf.hd, QKV = QD + 2 * KD;
  hipStream_t s = c.s;
  launch_embed_norm(act, tokens, m->w.emb, m->w.layers[0].g1, R, cf.D, cf.V, cf.eps, at<void>(c, c.L.x),
                    at<void>(c, c.L.u), s);
  for (int l = 0; l < cf.L; l++) {
    const dg_layer_weights& w = m->w.layers[l];
    inject_layer_input(c, l);
    if (l == cf.L - 1 && !head && !(taps && taps->qkv)) {
      // nothing downstream reads the last layer's queries or output: its K
      // and V columns only, straight into the cache
      CacheDst cd{kv->k[l], kv->v[l], kv->cap, T, 0, KD, cf.hd, cf.Hkv, lens};
      dense_gemm(c, GEMM_QKV_CACHE, at<void>(c, c.L.u), R, cf.D, w.wk, KD, w.wv, KD, nullptr, 2 * KD,
                 at<void>(c, c.L.qkv), 2 * KD, nullptr, &cd);
      break;
    }
    CacheDst cd{kv->k[l], kv->v[l], kv->cap, T, QD, KD, cf.hd, cf.Hkv, lens};
    dense_gemm(c, GEMM_QKV_CACHE, at<void>(c, c.L.u), R, cf.D, w.wq, QD, w.wk, KD, w.wv, QKV,
               at<void>(c, c.L.qkv), QKV, nullptr, &cd);
    if (taps) tap_copy(taps->qkv ? (char*)taps->qkv + (size_t)l * R * QKV * a : nullptr,
                       at<void>(c, c.L.qkv), (size_t)R * QKV * a, s);
    if (l == cf.L - 1 && !head) break;  // nothing downstream reads the last layer's output
    AttnArgsHost ah{act, at<void>(c, c.L.qkv), QKV, kv->k[l], kv->v[l], kv->cap, nullptr, nullptr,
                    B, T, cf.Hq, cf.Hkv, cf.hd, 1, lens, at<void>(c, c.L.o), at<void>(c, c.L.po),
                    at<float>(c, c.L.pml), c.L.part_cap};
    stage_event(taps, l, DG_STAGE_ATTN, 0, s);
    launch_attention(ah, s);
    stage_event(taps, l, DG_STAGE_ATTN, 1, s);
    if (taps) tap_copy(taps->attn ? (char*)taps->attn + (size_t)l * R * QD * a : nullptr,
                       at<void>(c, c.L.o), (size_t)R * QD * a, s);
    moe_block(c, l, l + 1 < cf.L ? m->w.layers[l + 1].g1 : m->w.gf);
  }
  if (head) {
    // next token of every row: the LM head over the final RMSNorm output
    const void* head_in = (taps && taps->inject_uf) ? taps->inject_uf : at<void>(c, c.L.u);
    stage_event(taps, cf.L - 1, DG_STAGE_HEAD, 0, s);
    const int nparts = launch_lmhead(act, head_in, R, cf.D, m->w.lm, cf.V, at<float>(c, c.L.lpm),
                                     at<int32_t>(c, c.L.lpi), at<float>(c, c.L.lps),
                                     taps ? taps->logits : nullptr, s);
    stage_event(taps, cf.L - 1, DG_STAGE_HEAD, 1, s);
    if (taps) tap_copy(taps->uf, at<void>(c, c.L.u), (size_t)R * cf.D * a, s);
    launch_lm_merge(at<float>(c, c.L.lpm), at<int32_t>(c, c.L.lpi), at<float>(c, c.L.lps), R, nparts,
                    argmax, conf, MergeNext{}, s);
  }
  dg_status st = check_hip();
  if (st != DG_OK) return st;
  for (int b = 0; b < B; b++) kv->len[b] += T;
  return DG_OK;
}

dg_status dg_kv_prefill(const dg_model* m, dg_kv* kv, const int32_t* tokens, int32_t B, int32_t T,
                        const dg_taps* taps, void* ws, size_t ws_bytes, void* stream) {
  return prefill(m, kv, tokens, B, T, taps, ws, ws_bytes, stream, nullptr, nullptr);
}

dg_status dg_decode_step(const dg_model* m, dg_kv* kv, const int32_t* tokens, int32_t B,
                         int32_t* argmax, float* conf, const dg_taps* taps, void* ws, size_t ws_bytes,
                         void* stream) {
  if (!argmax || !conf) return DG_ERR_INVALID;
  return prefill(m, kv, tokens, B, 1, taps, ws, ws_bytes, stream, argmax, conf);
}

// one pass; nx carries the between-pass work its last kernel takes over
static dg_status denoise(const dg_model* m, const dg_kv* kv, const int32_t* canvas, int32_t B,
                         int32_t N, int32_t* argmax, float* conf, const dg_taps* taps, void* ws,
                         size_t ws_bytes, void* stream, MergeNext nx, bool embed_next = false,
                         bool input_embedded = false) {
  if (!model_ok(m) || !kv || !kv->len || !canvas || !argmax || !conf || !ws) return DG_ERR_INVALID;
  if (B < 1 || B > DG_MAX_BATCH || N < 1) return DG_ERR_INVALID;
  const dg_config& cf = m->cfg;
  Lens lens{};
  bool any_prefix = false;
  int maxkeys = 0;
  for (int b = 0; b < B; b++) {
    if (kv->len[b] < 0 || (kv->len[b] > 0 && kv->len[b] > kv->cap)) return DG_ERR_INVALID;
    lens.v[b] = kv->len[b];
    any_prefix |= kv->len[b] > 0;
    maxkeys = kv->len[b] + N > maxkeys ? kv->len[b] + N : maxkeys;
  }
  if (any_prefix)
    for (int l = 0; l < cf.L; l++)
      if (!kv->k[l] || !kv->v[l]) return DG_ERR_INVALID;
  if ((long)B * N > (1L << 20)) return DG_ERR_UNSUPPORTED;
  const int R = B * N;
  Ctx c{m, (char*)ws, call_layout(cf, R, maxkeys, ws_bytes), R, taps, (hipStream_t)stream, true};
  if (c.L.total > ws_bytes) return DG_ERR_WORKSPACE;

  (void)hipGetLastError();
  const int act = cf.act_dtype == DG_BF16 ? ACT_BF16 : ACT_F32;
  const size_t a = esize(cf.act_dtype);
  const int QD = cf.Hq * cf.hd, KD = cf.Hkv * cf.hd, QKV = QD + 2 * KD;
  hipStream_t s = c.s;
  if (nx.rn.canvas) {
    c.zero0 = nx.rn.changed;
    c.zero1 = nx.rn.masked_left;
    c.nzero = B;
  }
  // the first layer's input: embedded here, or (input_embedded) written into
  // the workspace by the previous pass's last kernel
  if (!(nx.rn.canvas && input_embedded))
    launch_embed_norm(act, canvas, m->w.emb, m->w.layers[0].g1, R, cf.D, cf.V, cf.eps,
                      at<void>(c, c.L.x), at<void>(c, c.L.u), s);
  for (int l = 0; l < cf.L; l++) {
    const dg_layer_weights& w = m->w.layers[l];
    inject_layer_input(c, l);
    dense_gemm(c, GEMM_STORE, at<void>(c, c.L.u), R, cf.D, w.wq, QD, w.wk, KD, w.wv, QKV,
               at<void>(c, c.L.qkv), QKV, nullptr, nullptr);
    if (taps) tap_copy(taps->qkv ? (char*)taps->qkv + (size_t)l * R * QKV * a : nullptr,
                       at<void>(c, c.L.qkv), (size_t)R * QKV * a, s);
    const char* qkv = at<char>(c, c.L.qkv);
    AttnArgsHost ah{act, qkv, QKV, kv->k[l], kv->v[l], kv->cap, qkv + QD * a, qkv + (QD + KD) * a,
                    B, N, cf.Hq, cf.Hkv, cf.hd, 0, lens, at<void>(c, c.L.o), at<void>(c, c.L.po),
                    at<float>(c, c.L.pml), c.L.part_cap};
    stage_event(taps, l, DG_STAGE_ATTN, 0, s);
    launch_attention(ah, s);
    stage_event(taps, l, DG_STAGE_ATTN, 1, s);
    if (taps) tap_copy(taps->attn ? (char*)taps->attn + (size_t)l * R * QD * a : nullptr,
                       at<void>(c, c.L.o), (size_t)R * QD * a, s);
    moe_block(c, l, l + 1 < cf.L ? m->w.layers[l + 1].g1 : m->w.gf);
  }
  // head: logits tiles reduced to (max, argmax, sum exp), merged per row
  const void* head_in = (taps && taps->inject_uf) ? taps->inject_uf : at<void>(c, c.L.u);
  stage_event(taps, cf.L - 1, DG_STAGE_HEAD, 0, s);
  const int nparts = launch_lmhead(act, head_in, R, cf.D, m->w.lm, cf.V, at<float>(c, c.L.lpm),
                                   at<int32_t>(c, c.L.lpi), at<float>(c, c.L.lps),
                                   taps ? taps->logits : nullptr, s);
  stage_event(taps, cf.L - 1, DG_STAGE_HEAD, 1, s);
  if (taps) tap_copy(taps->uf, at<void>(c, c.L.u), (size_t)R * cf.D * a, s);
  nx.counts = at<int32_t>(c, c.L.cov);
  nx.L = cf.L;
  nx.E = cf.E;
  nx.rn.argmax = argmax;
  nx.rn.conf = conf;
  nx.rn.B = B;
  nx.rn.N = N;
  nx.rn.V = (uint32_t)cf.V;
  if (nx.rn.canvas && embed_next) {
    nx.act = act;
    nx.emb = m->w.emb;
    nx.g1 = m->w.layers[0].g1;
    nx.D = cf.D;
    nx.eps = cf.eps;
    nx.ex = at<void>(c, c.L.x);
    nx.eu = at<void>(c, c.L.u);
  }
  launch_lm_merge(at<float>(c, c.L.lpm), at<int32_t>(c, c.L.lpi), at<float>(c, c.L.lps), R, nparts,
                  argmax, conf, nx, s);
  return check_hip();
}

dg_status dg_denoise_pass(const dg_model* m, const dg_kv* kv, const int32_t* canvas, int32_t B,
                          int32_t N, int32_t* argmax, float* conf, const dg_taps* taps, void* ws,
                          size_t ws_bytes, void* stream) {
  return denoise(m, kv, canvas, B, N, argmax, conf, taps, ws, ws_bytes, stream, MergeNext{});
}

dg_status dg_denoise_pass_next(const dg_model* m, const dg_kv* kv, int32_t* canvas, int32_t B,
                               int32_t N, int32_t* argmax, float* conf, int32_t* touched,
                               const dg_renoise_args* next, const dg_taps* taps, void* ws,
                               size_t ws_bytes, void* stream) {
  MergeNext nx{};
  nx.touched = touched;
  if (next) {
    if (next->mode != DG_SAMPLER_UNIFORM && next->mode != DG_SAMPLER_MASKED) return DG_ERR_INVALID;
    // positions key the noise draws: required by uniform-state noise only
    if ((next->mode == DG_SAMPLER_UNIFORM && !next->pos0) || B < 1 || B > DG_MAX_BATCH)
      return DG_ERR_INVALID;
    if (!canvas || canvas == argmax || (const void*)canvas == (const void*)conf) return DG_ERR_INVALID;
    for (int b = 0; b < B; b++) {
      if (next->pos0 && next->pos0[b] < 0) return DG_ERR_INVALID;
      nx.rn.pos0.v[b] = next->pos0 ? next->pos0[b] : 0;
      nx.rn.req.v[b] = next->req_id ? next->req_id[b] : (uint32_t)b;
    }
    nx.rn.canvas = canvas;
    nx.rn.tau = next->tau;
    nx.rn.seed = next->seed;
    nx.rn.tag = next->pass_tag;
    nx.rn.mode = next->mode;
    nx.rn.mask_id = next->mask_id;
    nx.rn.final_pass = next->final_pass;
    nx.rn.changed = next->changed;
    nx.rn.masked_left = next->masked_left;
  }
  return denoise(m, kv, canvas, B, N, argmax, conf, taps, ws, ws_bytes, stream, nx,
                 next && next->embed_next, next && next->input_embedded);
}

dg_status dg_denoise_pass_next_noalloc(const dg_model* m, const dg_kv* kv, int32_t* canvas, int32_t B,
                                       int32_t N, int32_t* argmax, float* conf, int32_t* touched,
                                       const dg_renoise_args* next, const dg_taps* taps, void* stream) {
  if (!model_ok(m) || !kv || !kv->len || B < 1 || B > DG_MAX_BATCH || N < 1) return DG_ERR_INVALID;
  // reject, before touching the device, what the scratch cannot hold: the
  // fixed part of the carve (the attention split partials take what is left)
  if ((long)B * N > (1L << 20)) return DG_ERR_UNSUPPORTED;
  if (layout(m->cfg, B * N, 0).fixed > (size_t)DG_NOALLOC_SCRATCH_BYTES) return DG_ERR_WORKSPACE;
  dg_status st = DG_OK;
  void* ws = scratch_for_current_device(&st);
  if (!ws) return st;
  return dg_denoise_pass_next(m, kv, canvas, B, N, argmax, conf, touched, next, taps, ws,
                              (size_t)DG_NOALLOC_SCRATCH_BYTES, stream);
}

dg_status dg_renoise(int32_t* canvas, const int32_t* argmax, const float* conf, float tau,
                     uint64_t seed, uint32_t pass_tag, const int32_t* pos0, const uint32_t* req_id,
                     int32_t B, int32_t N, int32_t V, void* stream) {
  if (!canvas || !pos0 || B < 1 || B > DG_MAX_BATCH || N < 1 || V < 1) return DG_ERR_INVALID;
  if (conf && !argmax) return DG_ERR_INVALID;
  Lens p{};
  ReqIds r{};
  for (int b = 0; b < B; b++) {
    if (pos0[b] < 0) return DG_ERR_INVALID;
    p.v[b] = pos0[b];
    r.v[b] = req_id ? req_id[b] : (uint32_t)b;
  }
  (void)hipGetLastError();
  launch_renoise(canvas, argmax, conf, tau, seed, pass_tag, p, r, B, N, V, (hipStream_t)stream);
  return check_hip();
}

dg_status dg_canvas_update(int32_t* canvas, const int32_t* argmax, const float* conf,
                           const dg_renoise_args* a, int32_t B, int32_t N, int32_t V, void* stream) {
  if (!canvas || !a || B < 1 || B > DG_MAX_BATCH || N < 1 || V < 1) return DG_ERR_INVALID;
  if (conf && !argmax) return DG_ERR_INVALID;
  if (a->mode != DG_SAMPLER_UNIFORM && a->mode != DG_SAMPLER_MASKED) return DG_ERR_INVALID;
  RenoiseArgs r{};
  if (a->mode == DG_SAMPLER_UNIFORM && !a->pos0) return DG_ERR_INVALID;
  for (int b = 0; b < B; b++) {
    if (a->pos0 && a->pos0[b] < 0) return DG_ERR_INVALID;
    r.pos0.v[b] = a->pos0 ? a->pos0[b] : 0;
    r.req.v[b] = a->req_id ? a->req_id[b] : (uint32_t)b;
  }
  r.canvas = canvas;
  r.argmax = argmax;
  r.conf = conf;
  r.tau = a->tau;
  r.seed = a->seed;
  r.tag = a->pass_tag;
  r.B = B;
  r.N = N;
  r.V = (uint32_t)V;
  r.mode = a->mode;
  r.mask_id = a->mask_id;
  r.final_pass = a->final_pass;
  r.changed = a->changed;
  r.masked_left = a->masked_left;
  (void)hipGetLastError();
  launch_canvas_update(r, (hipStream_t)stream);
  return check_hip();
}

size_t dg_packed_bytes(int32_t rows, int32_t cols, int32_t dtype) {
  if (rows < 1 || cols < 1 ||
      (dtype != DG_F32 && dtype != DG_BF16 && dtype != DG_FP8E4M3 && dtype != DG_MXFP4))
    return 0;
  if (dtype == DG_MXFP4 && cols % 2) return 0;
  const size_t rowbytes = nbytes((size_t)cols, dtype);
  if (rowbytes % 128) return 0;
  return (size_t)((rows + 15) / 16) * 16 * rowbytes;
}

size_t dg_packed_mx_scale_bytes(int32_t rows, int32_t cols) {
  if (rows < 1 || cols < 1 || cols % 256) return 0;
  return (size_t)((rows + 15) / 16) * 16 * (cols / 32);
}

dg_status dg_pack_mx_scales(const void* src, void* dst, int32_t rows, int32_t cols, void* stream) {
  if (!src || !dst || src == dst) return DG_ERR_INVALID;
  if (dg_packed_mx_scale_bytes(rows, cols) == 0) return DG_ERR_INVALID;
  (void)hipGetLastError();
  launch_pack_mx_scales(src, dst, rows, cols / 32, (hipStream_t)stream);
  return check_hip();
}

dg_status dg_pack_weight(const void* src, void* dst, int32_t rows, int32_t cols, int32_t dtype,
                         void* stream) {
  if (!src || !dst || src == dst) return DG_ERR_INVALID;
  if (dg_packed_bytes(rows, cols, dtype) == 0) return DG_ERR_INVALID;
  if (nbytes((size_t)cols, dtype) > (size_t)INT32_MAX) return DG_ERR_UNSUPPORTED;
  (void)hipGetLastError();
  launch_pack(src, dst, rows, (int)nbytes((size_t)cols, dtype), (hipStream_t)stream);
  return check_hip();
}

dg_status dg_expert_coverage(const dg_model* m, const void* ws, size_t ws_bytes, int32_t* touched,
                             int32_t* counts, void* stream) {
  if (!model_ok(m) || !ws || !touched) return DG_ERR_INVALID;
  if ((size_t)m->cfg.L * m->cfg.E * 4 > ws_bytes) return DG_ERR_WORKSPACE;
  (void)hipGetLastError();
  launch_coverage((const int32_t*)ws, m->cfg.L, m->cfg.E, touched, counts, (hipStream_t)stream);
  return check_hip();
}

}  // extern "C"
