// Host engine and C ABI of the action-expert decision (see include/phx_expert.h).
//
// A handle owns three kinds of device memory, the buffer roles the pages
// describe ("FlashRT-PAI", section 3.4 and Appendix A.1):
//   static : re-tiled weights and the step-conditioning table (modulation of
//            every norm at every tau_k), written once at create;
//   state  : per-request prefix K/V caches (with room for the action rows),
//            prefix lengths and the decoder position table, written by
//            phx_expert_load_prefix_kv and read by every step;
//   working: the state x, residual stream h, sums of squares, q, o, the GeGLU
//            activation and split partials, reused by every layer.
// The step loop (S steps x NL layers) is captured once into a HIP graph whose
// nodes see only fixed addresses ("PhyAI", section 4.2 Graph replay).
#include "phx_expert.h"
#include "phx_internal.h"
#include "phx_decide.h"
#include "phx_tokens.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <cstdlib>
#include <string>
#include <algorithm>
#include <vector>

using namespace phx;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define PHX_HIP(call)                                                                                 \
  do {                                                                                                \
    hipError_t e_ = (call);                                                                           \
    if (e_ != hipSuccess) return fail(PHX_E_HIP, "%s failed: %s", #call, hipGetErrorString(e_));     \
  } while (0)

struct GemmPlan {
  int NT = 0, KT = 0, KSW = 1, NW = 4;
};

// One kernel launch of the step loop.
struct Node {
  int kind = 0, step = 0, layer = 0;
  uint64_t bytes = 0;  // algorithmic HBM bytes of one launch (weights and modulation rows)
  char name[32] = {0};
  GemmArgs g{};
  int nw = 1, pro = 0, epi = 0;
  AttnArgs at{};
  CombineArgs cb{};
};

// One kernel launch of the large-token plan.
enum TokOp : int { TOP_CVT = 0, TOP_NORM = 1, TOP_GEMM = 2, TOP_ATTN = 3, TOP_COMBINE = 4, TOP_MK_ATTN = 5,
                   TOP_MK_COMBINE = 6, TOP_MK_GEMM = 7 };

struct TokNode {
  int kind = 0, step = 0, layer = 0, op = 0, epi = 0;
  uint64_t bytes = 0;  // weights streamed plus activation rows read and written
  char name[32] = {0};
  tok::GemmT g{};
  tok::AttnT a{};
  AttnArgs mat{};     // TOP_MK_ATTN: the batched multi-query attention of the request caches
  CombineArgs mcb{};  // TOP_MK_COMBINE
  GemmArgs mg{};      // TOP_MK_GEMM: a small-M projection of the multi-kernel path (state width 32)
  int mk_nw = 1, mk_pro = 0, mk_epi = 0;
  // TOP_NORM / TOP_CVT
  int norm_kind = 0;  // 0 RMS, 1 LayerNorm
  const float* src = nullptr;
  const float* scale = nullptr;
  const float* shift = nullptr;
  float eps = 0.f;
  void* dst = nullptr;
  int cols = 0;
  int split = 0;  // TOP_NORM: write paired rows
};

GemmPlan make_plan(int K, int N, int target_wgs) {
  GemmPlan p;
  p.KT = K / TILE_K;
  p.NT = N / TILE_N;
  p.NW = (p.KT % 4 == 0) ? 4 : 1;
  p.KSW = 1;
  while (p.NT * p.KSW < target_wgs && p.KT % (p.KSW * 2 * p.NW) == 0) p.KSW *= 2;
  return p;
}


size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool is_device_pointer(const void* p) {
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged;
}

}  // namespace

struct phx_expert {
  phx_expert_config cfg{};
  // large-token plan: the MLP's two GEMMs take paired (hi + lo) bf16 activation rows
  bool pair_act = false;
  int dtype = 1;
  size_t esz = 2;
  int BM = 0, MT = 1, NTD = 0, ss_ld = 0, Ctot = 0, SMAX = 0, GMP = 0, QT = 1, NN = 0;
  size_t kv_layer = 0;  // elements of one layer's cache (all requests)
  GemmPlan p_in, p_qkv, p_o, p_gu, p_down, p_out;
  // static
  void* wt = nullptr;
  size_t off_in = 0, off_out = 0;
  std::vector<size_t> off_qkv, off_o, off_gu, off_down;
  float* modtab = nullptr;
  // 8-bit tier: int8 codes at the same element offsets as wt, per-column scales per matrix
  signed char* wq = nullptr;
  float* wsc = nullptr;
  std::vector<size_t> sc_qkv, sc_o, sc_gu, sc_down;
  // state
  void* kc = nullptr;
  void* vtc = nullptr;
  int* lens = nullptr;
  float2* rope = nullptr;
  std::vector<int> loaded;
  std::vector<int> lens_host;  // prefix lengths as last loaded (host copy)
  // working
  float* x = nullptr;
  float* h = nullptr;
  float* ss = nullptr;
  void* q = nullptr;
  void* o = nullptr;
  void* act = nullptr;
  float* part_o = nullptr;
  float2* part_ml = nullptr;
  float* gpart = nullptr;
  unsigned* counters = nullptr;
  // execution
  hipStream_t cap = nullptr;
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  int nodes = 0;
  std::vector<Node> node_list;
  std::vector<void*> allocs;
  // persistent decision kernel (pi0.5 shape, one request)
  bool persistent = false;
  dec::Args dargs{};
  void* arena = nullptr;      // exchange and control words, then the auxiliary tables (dec::AUX0)
  hipError_t scratch_rc = hipErrorNotInitialized;  // set-up of the device's static exchange memory
  int device = 0;             // the device the handle was created on
  void* kvt = nullptr;
  int n_chunks = 0;
  // large-token plan (a chunk of many rows, or the DiT-style block)
  bool tokens = false;
  bool batched = false;       // the plan for a batch of requests: large-token GEMMs, per-request caches
  int trows = 0;              // rows of the plan (batch * rows)
  int Mp = 0;                 // rows padded to tok::ROW_PAD
  int splits = 1;             // attention key splits
  int n_cu = 0;               // compute units of the device
  float* tpart = nullptr;     // GEMM split partials of the large-token plan
  // history update of the chunk plan: the commit pass, its graph, the window's position base and
  // staging for the window shift
  std::vector<TokNode> cnodes;
  hipGraph_t cgraph = nullptr;
  hipGraphExec_t cexec = nullptr;
  int pos_base = 0;
  void* tk_tmp = nullptr;
  void* tv_tmp = nullptr;
  // execution-state capsules: a pinned header staging area and the event of its last copy
  void* cap_host = nullptr;
  size_t cap_host_bytes = 0;
  hipEvent_t cap_event = nullptr;
  std::vector<TokNode> tnodes;
  void* xb = nullptr;         // bf16 state rows (input projection operand)
  void* nb = nullptr;         // bf16 normalised rows
  void* qkv = nullptr;        // bf16 query rows [Mp][H*Dh]
  int R = 0;                  // key rows per layer: prefix capacity plus the chunk, padded to 64
  void* tk = nullptr;         // key rows [layers][R][KVH*Dh]: prefix, then the chunk from row L
  void* tv = nullptr;         // values [layers][KVH][R*Dh] in the attention's fragment order
  float* po = nullptr;        // attention partials of the key splits
  float* pml = nullptr;
};

namespace {

void release(phx_expert* h) {
  if (!h) return;
  if (h->cap) (void)hipStreamSynchronize(h->cap);
  if (h->cap_event) {
    (void)hipEventSynchronize(h->cap_event);
    (void)hipEventDestroy(h->cap_event);
  }
  if (h->cap_host) (void)hipHostFree(h->cap_host);
  if (h->exec) (void)hipGraphExecDestroy(h->exec);
  if (h->graph) (void)hipGraphDestroy(h->graph);
  if (h->cexec) (void)hipGraphExecDestroy(h->cexec);
  if (h->cgraph) (void)hipGraphDestroy(h->cgraph);
  for (void* p : h->allocs) (void)hipFree(p);
  if (h->cap) (void)hipStreamDestroy(h->cap);
  delete h;
}

int alloc(phx_expert* h, void** p, size_t bytes, const char* what) {
  hipError_t e = hipMalloc(p, bytes < 256 ? 256 : bytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(PHX_E_NOMEM, "device allocation of %zu bytes for %s failed: %s", bytes, what, hipGetErrorString(e));
  }
  h->allocs.push_back(*p);
  return PHX_OK;
}

size_t weight_elems(const phx_expert_config* c) {
  const size_t D = c->width, A = c->state_dim, F = c->mlp_hidden, E = c->time_emb_dim, NL = c->layers;
  const size_t qkv = (size_t)(c->n_heads + 2 * c->n_kv_heads) * c->head_dim;
  const size_t hd = (size_t)c->n_heads * c->head_dim;
  if (c->block_kind == PHX_BLOCK_DIT) return NL * (D * qkv + hd * D + D * F + F * D) + NL * E * 6 * D;
  if (c->block_kind == PHX_BLOCK_PREFILL) return NL * (D * qkv + hd * D + D * 2 * F + F * D) + 2 * NL * D;
  const size_t per_layer = D * qkv + hd * D + D * 2 * F + F * D;
  return A * D + NL * per_layer + D * A + (2 * NL + 1) * E * 2 * D;
}

// Build the node list of one decision's step loop: every kernel launch, in
// order, with its arguments.  The graph is captured from this list, and the
// diagnostic entry point relaunches single entries of it.
int build_nodes(phx_expert* h) {
  const phx_expert_config& c = h->cfg;
  const int D = c.width, H = c.n_heads, Dh = c.head_dim, KVH = c.n_kv_heads, F = c.mlp_hidden, A = c.state_dim;
  const int M = c.rows, NL = c.layers;
  const int D2 = 2 * D;
  const size_t esz = h->esz;
  h->node_list.clear();
  auto gemm_node = [&](int kind, int k, int l, const GemmPlan& p, int pro, int epi, const GemmArgs& g, int K, int N,
                       const char* name) {
    Node nd{};
    nd.kind = kind; nd.step = k; nd.layer = l; nd.g = g; nd.nw = p.NW; nd.pro = pro; nd.epi = epi;
    nd.bytes = (g.Wq ? (uint64_t)K * N + (uint64_t)N * sizeof(float) : (uint64_t)K * N * esz) +
               (pro == PRO_NORM ? (uint64_t)D2 * sizeof(float) : 0);
    std::snprintf(nd.name, sizeof(nd.name), "%s", name);
    h->node_list.push_back(nd);
  };
  for (int k = 0; k < c.steps; ++k) {
    const float* mod_k = h->modtab + (size_t)k * h->NN * D2;
    // a1: input projection h = x . W_in
    {
      GemmArgs g{};
      g.W = (const char*)h->wt + h->off_in * esz;
      g.KT = h->p_in.KT; g.NT = h->p_in.NT; g.KSW = h->p_in.KSW; g.rows = h->BM;
      g.X = h->x; g.ldx = A;
      g.hout = h->h; g.ssout = h->ss; g.NTD = h->NTD; g.ss_ld = h->ss_ld; g.D = D;
      g.part = h->gpart; g.counters = h->counters;
      gemm_node(PHX_NODE_IN_PROJ, k, -1, h->p_in, PRO_XF32, EPI_STORE_H, g, A, D, "in_proj");
    }
    for (int l = 0; l < NL; ++l) {
      void* kc_l = (char*)h->kc + (size_t)l * h->kv_layer * esz;
      void* vtc_l = (char*)h->vtc + (size_t)l * h->kv_layer * esz;
      // a2: AdaRMSNorm + QKV + RoPE, k and v written into the action-row cache slots
      {
        GemmArgs g{};
        g.W = (const char*)h->wt + h->off_qkv[l] * esz;
        if (h->wq) { g.Wq = h->wq + h->off_qkv[l]; g.wsc = h->wsc + h->sc_qkv[l]; }
        g.KT = h->p_qkv.KT; g.NT = h->p_qkv.NT; g.KSW = h->p_qkv.KSW; g.rows = h->BM;
        g.h = h->h; g.ss = h->ss; g.NTD = h->NTD; g.ss_ld = h->ss_ld; g.D = D; g.eps = c.rms_eps;
        g.mod = mod_k + (size_t)(2 * l) * D2;
        g.part = h->gpart; g.counters = h->counters;
        g.q = h->q; g.kc = kc_l; g.vtc = vtc_l; g.lens = h->lens; g.rope = h->rope;
        g.M = M; g.H = H; g.KVH = KVH; g.Dh = Dh; g.Ctot = h->Ctot;
        gemm_node(PHX_NODE_NORM_QKV_ROPE, k, l, h->p_qkv, PRO_NORM, EPI_QKV, g, D, (H + 2 * KVH) * Dh,
                  "norm_qkv_rope");
      }
      // a3: split-KV multi-query attention, then the fixed-order combine
      {
        Node nd{};
        nd.kind = PHX_NODE_ATTENTION; nd.step = k; nd.layer = l;
        AttnArgs& at = nd.at;
        at.q = h->q; at.kc = kc_l; at.vtc = vtc_l; at.lens = h->lens;
        at.part_o = h->part_o; at.part_ml = h->part_ml;
        at.M = M; at.H = H; at.KVH = KVH; at.Dh = Dh; at.Ctot = h->Ctot; at.SMAX = h->SMAX; at.GMP = h->GMP;
        at.scale = (float)(1.0 / std::sqrt((double)Dh));
        nd.bytes = 0;  // depends on the loaded prefix lengths: computed by phx_expert_node_info
        std::snprintf(nd.name, sizeof(nd.name), "attention");
        h->node_list.push_back(nd);
        Node nc{};
        nc.kind = PHX_NODE_ATTN_COMBINE; nc.step = k; nc.layer = l;
        CombineArgs& cb = nc.cb;
        cb.part_o = h->part_o; cb.part_ml = h->part_ml; cb.lens = h->lens; cb.o = h->o;
        cb.M = M; cb.H = H; cb.KVH = KVH; cb.Dh = Dh; cb.SMAX = h->SMAX; cb.GMP = h->GMP;
        nc.bytes = 0;
        std::snprintf(nc.name, sizeof(nc.name), "attention_combine");
        h->node_list.push_back(nc);
      }
      // a4: out-projection + residual
      {
        GemmArgs g{};
        g.W = (const char*)h->wt + h->off_o[l] * esz;
        if (h->wq) { g.Wq = h->wq + h->off_o[l]; g.wsc = h->wsc + h->sc_o[l]; }
        g.KT = h->p_o.KT; g.NT = h->p_o.NT; g.KSW = h->p_o.KSW; g.rows = h->BM;
        g.X = h->o; g.ldx = H * Dh;
        g.hout = h->h; g.ssout = h->ss; g.NTD = h->NTD; g.ss_ld = h->ss_ld; g.D = D;
        g.part = h->gpart; g.counters = h->counters;
        gemm_node(PHX_NODE_OUT_PROJ_RESID, k, l, h->p_o, PRO_X, EPI_RESID, g, H * Dh, D, "out_proj_resid");
      }
      // a5: AdaRMSNorm + gate/up + GeGLU
      {
        GemmArgs g{};
        g.W = (const char*)h->wt + h->off_gu[l] * esz;
        if (h->wq) { g.Wq = h->wq + h->off_gu[l]; g.wsc = h->wsc + h->sc_gu[l]; }
        g.KT = h->p_gu.KT; g.NT = h->p_gu.NT; g.KSW = h->p_gu.KSW; g.rows = h->BM;
        g.h = h->h; g.ss = h->ss; g.NTD = h->NTD; g.ss_ld = h->ss_ld; g.D = D; g.eps = c.rms_eps;
        g.mod = mod_k + (size_t)(2 * l + 1) * D2;
        g.part = h->gpart; g.counters = h->counters;
        g.act = h->act; g.F = F;
        gemm_node(PHX_NODE_NORM_GATEUP_GEGLU, k, l, h->p_gu, PRO_NORM, EPI_GEGLU, g, D, 2 * F, "norm_gateup_geglu");
      }
      // a6: down-projection + residual
      {
        GemmArgs g{};
        g.W = (const char*)h->wt + h->off_down[l] * esz;
        if (h->wq) { g.Wq = h->wq + h->off_down[l]; g.wsc = h->wsc + h->sc_down[l]; }
        g.KT = h->p_down.KT; g.NT = h->p_down.NT; g.KSW = h->p_down.KSW; g.rows = h->BM;
        g.X = h->act; g.ldx = F;
        g.hout = h->h; g.ssout = h->ss; g.NTD = h->NTD; g.ss_ld = h->ss_ld; g.D = D;
        g.part = h->gpart; g.counters = h->counters;
        gemm_node(PHX_NODE_DOWN_PROJ_RESID, k, l, h->p_down, PRO_X, EPI_RESID, g, F, D, "down_proj_resid");
      }
    }
    // a7: final AdaRMSNorm + velocity projection + Euler update
    {
      GemmArgs g{};
      g.W = (const char*)h->wt + h->off_out * esz;
      g.KT = h->p_out.KT; g.NT = h->p_out.NT; g.KSW = h->p_out.KSW; g.rows = h->BM;
      g.h = h->h; g.ss = h->ss; g.NTD = h->NTD; g.ss_ld = h->ss_ld; g.D = D; g.eps = c.rms_eps;
      g.mod = mod_k + (size_t)(2 * NL) * D2;
      g.part = h->gpart; g.counters = h->counters;
      g.x = h->x; g.dt = c.dt; g.A = A;
      gemm_node(PHX_NODE_NORM_OUT_EULER, k, -1, h->p_out, PRO_NORM, EPI_EULER, g, D, A, "norm_out_proj_euler");
    }
  }
  return PHX_OK;
}

int launch_node(phx_expert* h, const Node& nd, hipStream_t s) {
  switch (nd.kind) {
    case PHX_NODE_ATTENTION:
      PHX_HIP(launch_attention(h->dtype, h->QT, nd.at, h->cfg.batch, s));
      break;
    case PHX_NODE_ATTN_COMBINE:
      PHX_HIP(launch_combine(h->dtype, nd.cb, h->cfg.batch, s));
      break;
    default:
      PHX_HIP(launch_gemm(h->dtype, nd.nw, h->MT, nd.pro, nd.epi, nd.g, s));
  }
  return PHX_OK;
}

// Enqueue one decision's step loop on stream s (graph capture or direct).
int launch_tok(phx_expert* h, const TokNode& nd, hipStream_t s);

int enqueue_steps(phx_expert* h, hipStream_t s) {
  if (h->tokens) {
    for (const TokNode& nd : h->tnodes) {
      int rc = launch_tok(h, nd, s);
      if (rc) return rc;
    }
    return PHX_OK;
  }
  for (const Node& nd : h->node_list) {
    int rc = launch_node(h, nd, s);
    if (rc) return rc;
  }
  return PHX_OK;
}

int mt_for_rows(int rows) {
  const int need = (rows + 15) / 16;
  if (need <= 1) return 1;
  if (need <= 2) return 2;
  if (need <= 4) return 4;
  return 10;
}


// The persistent decision kernel covers the pi0.5 expert shape for one
// request of up to 16 action rows in bf16; every other configuration runs the
// multi-kernel graph.
bool persistent_eligible(const phx_expert_config& c, const hipDeviceProp_t& prop) {
  if (c.flags & (PHX_FLAG_NO_GRAPH | PHX_FLAG_MULTI_KERNEL)) return false;
  if (c.block_kind != PHX_BLOCK_DECODER) return false;
  if (c.weight_dtype != PHX_DTYPE_BF16 || c.kv_dtype != PHX_DTYPE_BF16) return false;
  if (c.width != dec::D || c.n_heads != dec::H || c.head_dim != dec::DH || c.n_kv_heads != 1) return false;
  if (c.mlp_hidden != dec::F || c.state_dim != dec::A) return false;
  if (c.batch != 1 || c.rows < 1 || c.rows > dec::RP) return false;
  const int n_chunks = (c.prefix_capacity + dec::CHUNK - 1) / dec::CHUNK;
  if (n_chunks + 1 > dec::MAX_CHUNKS) return false;
  if (prop.multiProcessorCount != dec::G) return false;
  if (prop.maxSharedMemoryPerMultiProcessor < 160 * 1024) return false;
  // every arena must stay within the 32-bit range of a buffer resource
  if (dec::w_elems(c.layers) * 2ull >= (1ull << 32)) return false;
  const unsigned long long arena = (unsigned long long)dec::AUX_TAB +
                                   (unsigned long long)c.steps * dec::step_bytes(c.layers) +
                                   (unsigned long long)dec::G * dec::timeline_events(c.steps, c.layers) * 4ull;
  if (arena >= (1ull << 31)) return false;
  // the decision kernel's workgroups wait on each other, so all G of them must be resident at once:
  // one per compute unit, which its LDS ring and register budget have to allow
  int per_cu = 0;
  const hipError_t eo = dec::decide_occupancy(&per_cu);
  // its ranks inside an XCD need the workgroups dealt to the XCDs round-robin (probed once per process)
  bool placed = false;
  const hipError_t ep = eo == hipSuccess && per_cu >= 1 ? dec::decide_placement(&placed) : hipSuccess;
  if (std::getenv("PHX_VERBOSE"))
    std::fprintf(stderr, "phx: decision kernel occupancy %d per CU (%s), placement %s (%s)\n", per_cu,
                 hipGetErrorString(eo), placed ? "round-robin" : "other", hipGetErrorString(ep));
  if (eo != hipSuccess || per_cu < 1) {
    (void)hipGetLastError();
    return false;
  }
  if (ep != hipSuccess || !placed) {
    (void)hipGetLastError();
    return false;
  }
  return true;
}

int enqueue_persistent(phx_expert* h, hipStream_t s) {
  PHX_HIP(dec::launch_decide(h->dargs, s));
  PHX_HIP(dec::launch_decide_advance(h->dargs, s));
  return PHX_OK;
}

// Everything the persistent path needs after the weights are tiled: one
// arena holding the exchange and control words and then the auxiliary tables
// (prefix length, failure flag, state, position table, per-step scale and
// shift . W tables, timeline), the
// attention-tiled prefix K/V, and a two-node graph (decision kernel, tag
// advance).  Workgroup roles are a function of the workgroup index and the
// chunk count, computed in the kernel.
int create_persistent(phx_expert* h, const char* sb, hipStream_t stream, size_t mod_off_elems) {
  const phx_expert_config& c = h->cfg;
  const int S = c.steps, NL = c.layers, E = c.time_emb_dim;
  h->n_chunks = (c.prefix_capacity + dec::CHUNK - 1) / dec::CHUNK;
  const bool timeline = (c.flags & PHX_FLAG_TIMELINE) != 0;
  const size_t aux_bytes = dec::aux_bytes(S, NL, timeline);
  const size_t arena_bytes = (size_t)dec::AUX0 + aux_bytes;
  int rc;
  if ((rc = alloc(h, &h->arena, arena_bytes, "decision arena"))) return rc;
  PHX_HIP(hipMemsetAsync(h->arena, 0, arena_bytes, stream));
  char* aux = (char*)h->arena + dec::AUX0;
  h->rope = (float2*)(aux + dec::AUX_ROPE);
  h->lens = (int*)(aux + dec::AUX_LENS);
  h->x = (float*)(aux + dec::AUX_X);

  // step-conditioning table, then per step: the scales of every norm and the
  // shift . W products of the QKV, gate/up and velocity-head norms
  void* etab = nullptr;
  if ((rc = alloc(h, &etab, (size_t)S * E * sizeof(double), "time embedding"))) return rc;
  if ((rc = alloc(h, (void**)&h->modtab, (size_t)S * h->NN * 2 * dec::D * sizeof(float), "modulation table")))
    return rc;
  PHX_HIP(launch_time_embedding((double*)etab, S, E, c.tau0, c.dt, stream));
  PHX_HIP(launch_modulation(h->dtype, sb + mod_off_elems * h->esz, (const double*)etab, h->modtab, S, h->NN, E,
                            2 * dec::D, stream));
  PHX_HIP(dec::launch_scale_table(h->modtab, S, h->NN, aux, NL, stream));
  const long long lstride = (long long)dec::W_LAYER;
  const size_t ks = dec::step_bytes(NL) / sizeof(float);
  char* tab = aux + dec::AUX_TAB;
  // the 8-bit tier's scales: every layer's four projections, [NQKV][D][2F][D] per layer
  const bool w8 = h->wq != nullptr;
  if (w8 && (h->sc_qkv.size() != (size_t)NL || h->sc_qkv[0] != (size_t)dec::SC_QKV || h->sc_o[0] != (size_t)dec::SC_O ||
             h->sc_gu[0] != (size_t)dec::SC_GU || h->sc_down[0] != (size_t)dec::SC_DN ||
             (NL > 1 && h->sc_qkv[1] != (size_t)dec::SC_LAYER)))
    return fail(PHX_E_SHAPE, "int8 scale layout differs from the decision kernel's");
  const float* sc_qkv = w8 ? h->wsc + dec::SC_QKV : nullptr;
  const float* sc_gu = w8 ? h->wsc + dec::SC_GU : nullptr;
  PHX_HIP(dec::launch_shift_table(sb + h->off_qkv[0] * h->esz, lstride, h->modtab, h->NN, 2, 0, S, NL, dec::NQKV,
                                  COL_ROPE, dec::DH, sc_qkv, dec::SC_LAYER, (float*)(tab + dec::st_swqkv(NL)), ks,
                                  stream));
  PHX_HIP(dec::launch_shift_table(sb + h->off_gu[0] * h->esz, lstride, h->modtab, h->NN, 2, 1, S, NL, 2 * dec::F,
                                  COL_GEGLU, dec::F, sc_gu, dec::SC_LAYER, (float*)(tab + dec::st_swgu(NL)), ks,
                                  stream));
  PHX_HIP(dec::launch_shift_table(sb + h->off_out * h->esz, 0, h->modtab, h->NN, 0, 2 * NL, S, 1, dec::A, COL_IDENT,
                                  0, nullptr, 0, (float*)(tab + dec::st_swout(NL)), ks, stream));

  // attention-tiled prefix K/V
  const size_t kvt_bytes = (size_t)NL * h->n_chunks * 64 * dec::TILE_BYTES;
  if ((rc = alloc(h, &h->kvt, std::max(kvt_bytes, (size_t)dec::TILE_BYTES), "attention key/value tiles"))) return rc;
  PHX_HIP(hipMemsetAsync(h->kvt, 0, std::max(kvt_bytes, (size_t)dec::TILE_BYTES), stream));
  PHX_HIP(hipStreamSynchronize(stream));
  for (void* p : {etab, (void*)h->modtab})
    for (size_t i = 0; i < h->allocs.size(); ++i)
      if (h->allocs[i] == p) {
        (void)hipFree(p);
        h->allocs.erase(h->allocs.begin() + (long)i);
        break;
      }
  h->modtab = nullptr;

  // the kernel addresses the tiled weights with compile-time offsets
  if (h->off_in != 0 || h->off_qkv[0] != dec::W_QKV0 || h->off_o[0] != dec::W_O0 || h->off_gu[0] != dec::W_GU0 ||
      h->off_down[0] != dec::W_DN0 || h->off_out != dec::w_out(NL) ||
      (NL > 1 && h->off_qkv[1] - h->off_qkv[0] != dec::W_LAYER))
    return fail(PHX_E_SHAPE, "tiled weight layout differs from the decision kernel's");

  dec::Args& a = h->dargs;
  a.wt = h->wt;
  a.kvt = h->kvt;
  a.ex = h->arena;
  a.aux = aux;
  a.wt_bytes = (unsigned)(dec::w_elems(NL) * 2ull);
  a.kvt_bytes = (unsigned)kvt_bytes;
  a.aux_bytes = (unsigned)aux_bytes;
  a.wq = w8 ? h->wq : nullptr;
  a.wsc = w8 ? h->wsc : nullptr;
  a.wq_bytes = w8 ? (unsigned)dec::w_elems(NL) : 0u;
  a.wsc_bytes = w8 ? (unsigned)((size_t)NL * dec::SC_LAYER * sizeof(float)) : 0u;
  // the device's static exchange memory, for decisions that may not allocate
  // (phx_expert_decide_noalloc); the handle's own decisions do not need it
  h->scratch_rc = dec::decide_scratch_setup();
  if (h->scratch_rc != hipSuccess) (void)hipGetLastError();
  a.tl = timeline ? 1u : 0u;
  a.S = S;
  a.NL = NL;
  a.R = c.rows;
  a.n_chunks = h->n_chunks;
  a.dt = c.dt;
  a.eps = c.rms_eps;

  // diagnostics node list: the decision kernel (with its tag advance)
  h->node_list.clear();
  {
    Node nd{};
    nd.kind = PHX_NODE_DECISION;
    nd.step = -1;
    nd.layer = -1;
    std::snprintf(nd.name, sizeof(nd.name), "decision_kernel");
    h->node_list.push_back(nd);
    Node na{};
    na.kind = PHX_NODE_TAG_ADVANCE;
    na.step = -1;
    na.layer = -1;
    std::snprintf(na.name, sizeof(na.name), "tag_advance");
    h->node_list.push_back(na);
  }
  h->nodes = 2;
  PHX_HIP(hipStreamBeginCapture(h->cap, hipStreamCaptureModeThreadLocal));
  rc = enqueue_persistent(h, h->cap);
  hipGraph_t g = nullptr;
  hipError_t e = hipStreamEndCapture(h->cap, &g);
  if (rc) {
    if (g) (void)hipGraphDestroy(g);
    return rc;
  }
  if (e != hipSuccess) return fail(PHX_E_HIP, "hipStreamEndCapture failed: %s", hipGetErrorString(e));
  h->graph = g;
  PHX_HIP(hipGraphInstantiate(&h->exec, h->graph, nullptr, nullptr, 0));
  return PHX_OK;
}


bool uses_tokens(const phx_expert_config& c) {
  return c.block_kind != PHX_BLOCK_DECODER || (long long)c.rows * c.batch > 160;
}

// A bf16 batch of 65..160 rows: the large-token GEMMs on all rows at once
// (each weight byte serves every request) with the per-request caches and the
// batched multi-query attention of the multi-kernel path.
bool uses_batched(const phx_expert_config& c) {
  const long long rows = (long long)c.rows * c.batch;
  return c.block_kind == PHX_BLOCK_DECODER && c.weight_dtype == PHX_DTYPE_BF16 && rows > 64 && rows <= 160 &&
         !(c.flags & (PHX_FLAG_MULTI_KERNEL | PHX_FLAG_WEIGHTS_INT8));
}

int launch_tok(phx_expert* h, const TokNode& nd, hipStream_t s) {
  const int M = h->trows;
  switch (nd.op) {
    case TOP_CVT:
      PHX_HIP(tok::launch_tcvt(nd.src, nd.dst, M, h->Mp, nd.cols, s));
      break;
    case TOP_NORM:
      PHX_HIP(tok::launch_tnorm(nd.norm_kind, nd.src, nd.scale, nd.shift, nd.eps, nd.dst, M, h->Mp, nd.cols,
                                nd.split, s));
      break;
    case TOP_GEMM:
      PHX_HIP(tok::launch_tgemm(nd.epi, nd.g, s));
      break;
    case TOP_ATTN:
      PHX_HIP(tok::launch_tattn(nd.a, s));
      break;
    case TOP_COMBINE:
      PHX_HIP(tok::launch_tcombine(nd.a, s));
      break;
    case TOP_MK_ATTN:
      PHX_HIP(launch_attention(1, h->QT, nd.mat, h->cfg.batch, s));
      break;
    case TOP_MK_COMBINE:
      PHX_HIP(launch_combine(1, nd.mcb, h->cfg.batch, s));
      break;
    case TOP_MK_GEMM:
      PHX_HIP(launch_gemm(1, nd.mk_nw, h->MT, nd.mk_pro, nd.mk_epi, nd.mg, s));
      break;
    default:
      return fail(PHX_E_INVALID, "unknown token-plan op %d", nd.op);
  }
  return PHX_OK;
}

// The launches of one large-token decision.  Decoder block (a chunk of rows
// over a prefix cache): per Euler step the state goes to bf16, the input
// projection, then per layer RMS norm, QKV with RoPE, attention over prefix
// plus chunk keys, out-projection + residual, RMS norm, gate/up with GeGLU,
// down-projection + residual; then the final norm and the velocity
// projection with the Euler update.  DiT-style block: per block LayerNorm
// with shift and scale, QKV, attention over the tokens, gated out-projection
// residual, LayerNorm, up with GELU, gated down-projection residual.
int build_tok_nodes(phx_expert* h, bool commit = false) {
  const phx_expert_config& c = h->cfg;
  const bool dit = c.block_kind == PHX_BLOCK_DIT;
  const bool prefill = c.block_kind == PHX_BLOCK_PREFILL;
  const int D = c.width, H = c.n_heads, KVH = c.n_kv_heads, F = c.mlp_hidden, A = c.state_dim, M = h->trows;
  const int NL = c.layers, Dh = c.head_dim;
  const int HD = H * Dh, NQKV = (H + 2 * KVH) * Dh, kvd = KVH * Dh;
  const int Mp = h->Mp;
  // paired activation rows (hi + lo bf16) for the MLP's two GEMMs, gate/up and down, and for the prefill's
  // QKV (its keys and values are the prefill's output).  Elsewhere the QKV input stays plain bf16, whose
  // rounding measured well inside the bar: one DiT-style block 9.7e-3 with only the MLP paired against
  // 7.8e-3 with QKV paired too, at 7.83 against 8.60 ms per step; the prefill's 18-layer cache reached
  // 2.2e-2 with a plain QKV input
  const int pm = h->pair_act ? 1 : 0;
  const int pq = prefill ? pm : 0;
  h->tnodes.clear();
  auto name_of = [](TokNode& nd, const char* name) { std::snprintf(nd.name, sizeof(nd.name), "%s", name); };
  // pair: bit 0 = the activation rows are paired (hi + lo), bit 1 = the GELU/GeGLU output is written paired
  auto gemm = [&](int kind, int k, int l, int epi, const void* a, size_t w_off, int K, int N, void* out, int ldo,
                  const float* gate, const char* name, int pair = 0) {
    TokNode nd{};
    nd.kind = kind; nd.step = k; nd.layer = l; nd.op = TOP_GEMM; nd.epi = epi;
    tok::GemmT& g = nd.g;
    g.a = a; g.w = (const char*)h->wt + w_off * 2; g.out = out; g.gate = gate; g.rope = h->rope;
    g.rot_cols = dit ? 0 : (H + KVH) * Dh; g.dt = c.dt; g.M = M; g.Mp = Mp; g.N = N;
    g.wsh = pair & 1;
    g.K = K << g.wsh;
    g.osplit = (pair >> 1) & 1;
    g.ldo = ldo << g.osplit;
    tok::plan_gemm(g, h->n_cu);
    std::snprintf(nd.name, sizeof(nd.name), "%s %s/%d%s", name, tok::tile_name(g.tile), g.splits,
                  g.wsh ? " pair" : "");
    const int out_cols = (epi == tok::EP_GEGLU ? N / 2 : N) << g.osplit;
    const int out_esz = (epi == tok::EP_RESID || epi == tok::EP_EULER || epi == tok::EP_F32) ? 4 : 2;
    const uint64_t rmw = (epi == tok::EP_RESID || epi == tok::EP_EULER) ? 2 : 1;
    nd.bytes = (uint64_t)K * N * 2 + (uint64_t)M * g.K * 2 + rmw * (uint64_t)M * out_cols * out_esz +
               (gate ? (uint64_t)N * 4 : 0);
    h->tnodes.push_back(nd);
  };
  auto norm = [&](int k, int l, int kind, const float* scale, const float* shift, const char* name, int split = 0) {
    // right after a residual GEMM whose k splits end in a reduction launch, the norm runs in that launch
    if (!h->tnodes.empty()) {
      TokNode& prev = h->tnodes.back();
      tok::GemmT& pg = prev.g;
      if (prev.op == TOP_GEMM && prev.epi == tok::EP_RESID && pg.splits > 1 && pg.out == h->h && pg.N == D &&
          pg.ldo == D && D <= 256 * 16) {
        pg.nrm_on = 1; pg.nrm_kind = kind; pg.nrm_scale = scale; pg.nrm_shift = shift; pg.nrm_eps = c.rms_eps;
        pg.nrm_out = h->nb; pg.nrm_split = split;
        prev.bytes += (uint64_t)Mp * D * 2 * (split ? 2 : 1) + 2ull * D * 4;
        const size_t len = std::strlen(prev.name);
        std::snprintf(prev.name + len, sizeof(prev.name) - len, "+norm");
        return;
      }
    }
    TokNode nd{};
    nd.kind = PHX_NODE_ROW_NORM; nd.step = k; nd.layer = l; nd.op = TOP_NORM;
    nd.norm_kind = kind; nd.src = h->h; nd.scale = scale; nd.shift = shift; nd.eps = c.rms_eps; nd.dst = h->nb;
    nd.cols = D; nd.split = split;
    nd.bytes = (uint64_t)M * D * 4 + (uint64_t)Mp * D * 2 * (split ? 2 : 1) + 2ull * D * 4;
    name_of(nd, name);
    h->tnodes.push_back(nd);
  };
  const int R = h->R;
  auto layer_k = [&](int l) { return (char*)h->tk + (dit ? 0 : (size_t)l * R * kvd * 2); };
  auto layer_v = [&](int l) { return (char*)h->tv + (dit ? 0 : (size_t)l * R * kvd * 2); };
  auto qkv = [&](int k, int l, const char* name) {
    gemm(PHX_NODE_QKV, k, l, h->batched ? tok::EP_QKV_CACHE : tok::EP_QKV, h->nb, h->off_qkv[l], D, NQKV, h->qkv,
         HD, nullptr, name, pq);
    tok::GemmT& g = h->tnodes.back().g;
    g.kj = layer_k(l); g.vt = layer_v(l); g.lens = dit ? nullptr : h->lens; g.H = H; g.KVH = KVH; g.nj = R / 32;
    g.hd = Dh;
    // the batched plan's QKV (at most 160 rows) runs without k splits: its split reduction would be a launch
    // of its own, since the cache epilogue cannot ride on a norm, and costs more than the extra
    // workgroups gain (16-request rollout: 12.94 -> 12.62 ms)
    if (h->batched && g.splits > 1) {
      g.splits = 1;
      std::snprintf(h->tnodes.back().name, sizeof(h->tnodes.back().name), "%s %s/1", name, tok::tile_name(g.tile));
    }
    if (h->batched) {
      g.req_rows = c.rows; g.Ctot = h->Ctot;
      g.kc = (char*)h->kc + (size_t)l * h->kv_layer * 2;
      g.vtc = (char*)h->vtc + (size_t)l * h->kv_layer * 2;
    }
  };
  auto attention = [&](int k, int l) {
    if (h->batched) {
      TokNode nd{};
      nd.kind = PHX_NODE_ATTENTION; nd.step = k; nd.layer = l; nd.op = TOP_MK_ATTN;
      AttnArgs& at = nd.mat;
      at.q = h->qkv; at.kc = (char*)h->kc + (size_t)l * h->kv_layer * 2;
      at.vtc = (char*)h->vtc + (size_t)l * h->kv_layer * 2; at.lens = h->lens;
      at.part_o = h->part_o; at.part_ml = h->part_ml;
      at.M = c.rows; at.H = H; at.KVH = KVH; at.Dh = Dh; at.Ctot = h->Ctot; at.SMAX = h->SMAX; at.GMP = h->GMP;
      at.scale = (float)(1.0 / std::sqrt((double)Dh));
      name_of(nd, "attention");
      h->tnodes.push_back(nd);
      TokNode nc{};
      nc.kind = PHX_NODE_ATTN_COMBINE; nc.step = k; nc.layer = l; nc.op = TOP_MK_COMBINE;
      CombineArgs& cb = nc.mcb;
      cb.part_o = h->part_o; cb.part_ml = h->part_ml; cb.lens = h->lens; cb.o = h->o;
      cb.M = c.rows; cb.H = H; cb.KVH = KVH; cb.Dh = Dh; cb.SMAX = h->SMAX; cb.GMP = h->GMP;
      name_of(nc, "attention_combine");
      h->tnodes.push_back(nc);
      return;
    }
    TokNode nd{};
    nd.kind = PHX_NODE_ATTENTION; nd.step = k; nd.layer = l; nd.op = TOP_ATTN;
    tok::AttnT& a = nd.a;
    a.q = h->qkv; a.ldq = HD; a.kj = layer_k(l); a.vt = layer_v(l); a.lens = dit ? nullptr : h->lens; a.R = R;
    a.M = M; a.H = H; a.KVH = KVH; a.o = h->o; a.po = h->po; a.pml = h->pml; a.splits = h->splits;
    a.scale = (float)(1.0 / std::sqrt((double)Dh));
    a.hd = Dh;
    a.causal = prefill ? 1 : 0;
    name_of(nd, prefill ? "causal_attention" : "attention");
    h->tnodes.push_back(nd);
    if (h->splits > 1) {
      TokNode cb = nd;
      cb.kind = PHX_NODE_ATTN_COMBINE; cb.op = TOP_COMBINE;
      cb.bytes = (uint64_t)h->splits * M * (HD + 2 * H) * 4 + (uint64_t)M * HD * 2;
      name_of(cb, "attention_combine");
      h->tnodes.push_back(cb);
    }
  };
  if (dit) {
    for (int l = 0; l < NL; ++l) {
      const float* mod = h->modtab + (size_t)l * 6 * D;  // shift, scale, gate (attention), then (MLP)
      norm(0, l, 1, mod + D, mod, "layernorm_attn", pq);
      qkv(0, l, "qkv");
      attention(0, l);
      gemm(PHX_NODE_OUT_PROJ_RESID, 0, l, tok::EP_RESID, h->o, h->off_o[l], HD, D, h->h, D, mod + 2 * D,
           "out_proj_gated_resid");
      norm(0, l, 1, mod + 4 * D, mod + 3 * D, "layernorm_mlp", pm);
      gemm(PHX_NODE_GATEUP, 0, l, tok::EP_GELU, h->nb, h->off_gu[l], D, F, h->act, F, nullptr, "up_gelu", pm * 3);
      gemm(PHX_NODE_DOWN_PROJ_RESID, 0, l, tok::EP_RESID, h->act, h->off_down[l], F, D, h->h, D, mod + 5 * D,
           "down_proj_gated_resid", pm);
    }
    return PHX_OK;
  }
  if (prefill) {
    // the prefix prefill: per layer RMS norm with the layer's gains, QKV with RoPE (the layer's keys and
    // values land in rows 0.. of its key rows and value fragments), causal attention, out-projection +
    // residual, RMS norm, gate/up with GeGLU, down-projection + residual; the last layer writes its
    // cache and needs nothing after its QKV
    for (int l = 0; l < NL; ++l) {
      const float* m1 = h->modtab + (size_t)(2 * l) * 2 * D;
      const float* m2 = h->modtab + (size_t)(2 * l + 1) * 2 * D;
      norm(0, l, 0, m1, m1 + D, "rmsnorm_attn", pq);
      qkv(0, l, "qkv_rope");
      if (l + 1 == NL) break;
      attention(0, l);
      gemm(PHX_NODE_OUT_PROJ_RESID, 0, l, tok::EP_RESID, h->o, h->off_o[l], HD, D, h->h, D, nullptr,
           "out_proj_resid");
      norm(0, l, 0, m2, m2 + D, "rmsnorm_mlp", pm);
      gemm(PHX_NODE_GATEUP, 0, l, tok::EP_GEGLU, h->nb, h->off_gu[l], D, 2 * F, h->act, F, nullptr, "gateup_geglu",
           pm * 3);
      gemm(PHX_NODE_DOWN_PROJ_RESID, 0, l, tok::EP_RESID, h->act, h->off_down[l], F, D, h->h, D, nullptr,
           "down_proj_resid", pm);
    }
    return PHX_OK;
  }
  const int NN = 2 * NL + 1;
  if (commit) {
    // the history update: one pass of the layer stack over the committed chunk at the end flow time
    // (modulation row S); each layer's QKV writes the chunk's keys and values after the L cached rows,
    // and the last layer needs nothing after its QKV
    const int k = c.steps;
    const float* mod_k = h->modtab + (size_t)k * NN * 2 * D;
    TokNode nd{};
    nd.kind = PHX_NODE_STATE_CVT; nd.step = k; nd.layer = -1; nd.op = TOP_CVT;
    nd.src = h->x; nd.dst = h->xb; nd.cols = A;
    name_of(nd, "state_to_bf16");
    h->tnodes.push_back(nd);
    gemm(PHX_NODE_IN_PROJ, k, -1, tok::EP_F32, h->xb, h->off_in, A, D, h->h, D, nullptr, "in_proj");
    for (int l = 0; l < NL; ++l) {
      const float* m1 = mod_k + (size_t)(2 * l) * 2 * D;
      const float* m2 = mod_k + (size_t)(2 * l + 1) * 2 * D;
      norm(k, l, 0, m1, m1 + D, "rmsnorm_attn", pq);
      qkv(k, l, "qkv_rope");
      if (l + 1 == NL) break;
      attention(k, l);
      gemm(PHX_NODE_OUT_PROJ_RESID, k, l, tok::EP_RESID, h->o, h->off_o[l], HD, D, h->h, D, nullptr,
           "out_proj_resid");
      norm(k, l, 0, m2, m2 + D, "rmsnorm_mlp", pm);
      gemm(PHX_NODE_GATEUP, k, l, tok::EP_GEGLU, h->nb, h->off_gu[l], D, 2 * F, h->act, F, nullptr, "gateup_geglu",
           pm * 3);
      gemm(PHX_NODE_DOWN_PROJ_RESID, k, l, tok::EP_RESID, h->act, h->off_down[l], F, D, h->h, D, nullptr,
           "down_proj_resid", pm);
    }
    return PHX_OK;
  }
  // the batched plan keeps the state-width projections (K or N = state_dim, often 32) on the small-M GEMM
  auto mk_gemm = [&](int kind, int k, const GemmPlan& p, int pro, int epi, const GemmArgs& g, uint64_t bytes,
                     const char* name) {
    TokNode nd{};
    nd.kind = kind; nd.step = k; nd.layer = -1; nd.op = TOP_MK_GEMM; nd.mg = g;
    nd.mk_nw = p.NW; nd.mk_pro = pro; nd.mk_epi = epi; nd.bytes = bytes;
    name_of(nd, name);
    h->tnodes.push_back(nd);
  };
  for (int k = 0; k < c.steps; ++k) {
    const float* mod_k = h->modtab + (size_t)k * NN * 2 * D;  // per norm: scale, then shift
    if (h->batched) {
      GemmArgs g{};
      g.W = (const char*)h->wt + h->off_in * 2;
      g.KT = h->p_in.KT; g.NT = h->p_in.NT; g.KSW = h->p_in.KSW; g.rows = M;
      g.X = h->x; g.ldx = A;
      g.hout = h->h; g.ssout = h->ss; g.NTD = h->NTD; g.ss_ld = h->ss_ld; g.D = D;
      g.part = h->gpart; g.counters = h->counters;
      mk_gemm(PHX_NODE_IN_PROJ, k, h->p_in, PRO_XF32, EPI_STORE_H, g, (uint64_t)A * D * 2, "in_proj");
    } else {
      TokNode nd{};
      nd.kind = PHX_NODE_STATE_CVT; nd.step = k; nd.layer = -1; nd.op = TOP_CVT;
      nd.src = h->x; nd.dst = h->xb; nd.cols = A;
      nd.bytes = (uint64_t)M * A * 4 + (uint64_t)Mp * A * 2;
      name_of(nd, "state_to_bf16");
      h->tnodes.push_back(nd);
      gemm(PHX_NODE_IN_PROJ, k, -1, tok::EP_F32, h->xb, h->off_in, A, D, h->h, D, nullptr, "in_proj");
    }
    for (int l = 0; l < NL; ++l) {
      const float* m1 = mod_k + (size_t)(2 * l) * 2 * D;
      const float* m2 = mod_k + (size_t)(2 * l + 1) * 2 * D;
      norm(k, l, 0, m1, m1 + D, "rmsnorm_attn", pq);
      qkv(k, l, "qkv_rope");
      attention(k, l);
      gemm(PHX_NODE_OUT_PROJ_RESID, k, l, tok::EP_RESID, h->o, h->off_o[l], HD, D, h->h, D, nullptr,
           "out_proj_resid");
      norm(k, l, 0, m2, m2 + D, "rmsnorm_mlp", pm);
      gemm(PHX_NODE_GATEUP, k, l, tok::EP_GEGLU, h->nb, h->off_gu[l], D, 2 * F, h->act, F, nullptr, "gateup_geglu",
           pm * 3);
      gemm(PHX_NODE_DOWN_PROJ_RESID, k, l, tok::EP_RESID, h->act, h->off_down[l], F, D, h->h, D, nullptr,
           "down_proj_resid", pm);
    }
    const float* mf = mod_k + (size_t)(2 * NL) * 2 * D;
    norm(k, -1, 0, mf, mf + D, "rmsnorm_final");
    if (h->batched) {
      GemmArgs g{};
      g.W = (const char*)h->wt + h->off_out * 2;
      g.KT = h->p_out.KT; g.NT = h->p_out.NT; g.KSW = h->p_out.KSW; g.rows = M;
      g.X = h->nb; g.ldx = D; g.D = D;
      g.part = h->gpart; g.counters = h->counters;
      g.x = h->x; g.dt = c.dt; g.A = A;
      mk_gemm(PHX_NODE_OUT_EULER, k, h->p_out, PRO_X, EPI_EULER, g, (uint64_t)D * A * 2, "out_proj_euler");
    } else {
      gemm(PHX_NODE_OUT_EULER, k, -1, tok::EP_EULER, h->nb, h->off_out, D, A, h->x, A, nullptr, "out_proj_euler");
    }
  }
  return PHX_OK;
}

// Captures a node list into a graph on the handle's capture stream.
int capture_tok(phx_expert* h, const std::vector<TokNode>& list, hipGraph_t* graph, hipGraphExec_t* exec) {
  PHX_HIP(hipStreamBeginCapture(h->cap, hipStreamCaptureModeThreadLocal));
  int rc = PHX_OK;
  for (const TokNode& nd : list)
    if ((rc = launch_tok(h, nd, h->cap))) break;
  hipGraph_t g = nullptr;
  hipError_t e = hipStreamEndCapture(h->cap, &g);
  if (rc) {
    if (g) (void)hipGraphDestroy(g);
    return rc;
  }
  if (e != hipSuccess) return fail(PHX_E_HIP, "hipStreamEndCapture failed: %s", hipGetErrorString(e));
  *graph = g;
  PHX_HIP(hipGraphInstantiate(exec, g, nullptr, nullptr, 0));
  return PHX_OK;
}

// Set-up of the large-token plan after the weights are tiled: modulation
// table, state and working rows, the prefix cache, and the captured graph.
int create_tokens(phx_expert* h, const char* sb, hipStream_t stream, size_t mod_off) {
  const phx_expert_config& c = h->cfg;
  const bool dit = c.block_kind == PHX_BLOCK_DIT;
  const bool prefill = c.block_kind == PHX_BLOCK_PREFILL;
  h->trows = c.rows * c.batch;
  const int D = c.width, H = c.n_heads, KVH = c.n_kv_heads, F = c.mlp_hidden, A = c.state_dim, M = h->trows;
  const int NL = c.layers, S = c.steps, E = c.time_emb_dim, C = c.prefix_capacity;
  const int HD = H * c.head_dim, kvd = KVH * c.head_dim;
  const int Mp = (M + tok::ROW_PAD - 1) / tok::ROW_PAD * tok::ROW_PAD;
  h->Mp = Mp;
  // paired activations (the inputs of QKV, gate/up and down: both norms' rows and the MLP activation):
  // the default of the DiT-style block (its gated MLP branch carries the largest rounding of bf16
  // activations into the residual stream), of the batched plan and of the prefill (these roundings are
  // most of what a decision, or an 18-layer cache, accumulates); opt-in for the video-action chunk
  h->pair_act = !(c.flags & PHX_FLAG_BF16_ACT) && (dit || h->batched || prefill || (c.flags & PHX_FLAG_PAIRED_ACT));
  int rc;
  // modulation: decoder [S][2NL+1][2D] (scale | shift per norm); DiT [NL][6D] at tau0
  // (the decoder gets one more step row, at the end flow time tau0 + S dt, for the history update)
  // (the prefill's norms take its gains: [2NL][2D] rows of scale = g, shift = 0)
  const int MS = dit ? 1 : S + 1, NN = dit ? NL : 2 * NL + 1, MW = dit ? 6 * D : 2 * D;
  void* etab = nullptr;
  if (prefill) {
    const size_t ng = (size_t)2 * NL * D;
    std::vector<uint16_t> gb(ng);
    std::vector<float> tab(2 * ng, 0.f);
    PHX_HIP(hipMemcpyAsync(gb.data(), sb + mod_off * 2, ng * 2, hipMemcpyDeviceToHost, stream));
    PHX_HIP(hipStreamSynchronize(stream));
    for (size_t n = 0; n < (size_t)2 * NL; ++n)
      for (int d = 0; d < D; ++d) {
        const uint32_t u = (uint32_t)gb[n * D + d] << 16;  // bf16 -> f32 is exact
        std::memcpy(&tab[n * 2 * D + d], &u, 4);
      }
    if ((rc = alloc(h, (void**)&h->modtab, tab.size() * sizeof(float), "norm gains"))) return rc;
    PHX_HIP(hipMemcpyAsync(h->modtab, tab.data(), tab.size() * sizeof(float), hipMemcpyHostToDevice, stream));
    PHX_HIP(hipStreamSynchronize(stream));
  } else {
    if ((rc = alloc(h, &etab, (size_t)MS * E * sizeof(double), "time embedding"))) return rc;
    if ((rc = alloc(h, (void**)&h->modtab, (size_t)MS * NN * MW * sizeof(float), "modulation table"))) return rc;
    PHX_HIP(launch_time_embedding((double*)etab, MS, E, c.tau0, c.dt, stream));
    PHX_HIP(launch_modulation(1, sb + mod_off * 2, (const double*)etab, h->modtab, MS, NN, E, MW, stream));
  }

  // key rows: the prefix capacity plus the chunk, padded to whole 64-key blocks
  h->R = (C + M + 63) / 64 * 64;
  const int R = h->R;
  // attention key splits: enough workgroups to cover the chip, at least two key blocks per split
  const int qw = tok::attn_queries_per_wg(M, c.head_dim);
  const long long q_wgs = (long long)((M + qw - 1) / qw) * H;
  const int max_blocks = R / 64;
  h->splits = 1;
  while (q_wgs * h->splits < 256 && max_blocks / (h->splits * 2) >= 2) h->splits *= 2;

  struct Buf { void** p; size_t bytes; const char* what; };
  std::vector<Buf> bufs = {
      {(void**)&h->h, (size_t)Mp * D * 4, "residual rows"},
      {&h->nb, (size_t)Mp * D * 2 * (h->pair_act ? 2 : 1), "normalised rows"},
      {&h->qkv, (size_t)Mp * HD * 2, "query rows"},
      {&h->o, (size_t)Mp * HD * 2, "attention output rows"},
      {&h->act, (size_t)Mp * F * 2 * (h->pair_act ? 2 : 1), "MLP activation rows"},
  };
  if (h->batched) {
    // the multi-kernel path's per-request caches, lengths, position table and attention partials
    h->splits = 1;
    const size_t cache_bytes = (size_t)NL * h->kv_layer * 2;
    const size_t part_rows = (size_t)c.batch * KVH * h->SMAX * h->GMP;
    bufs.push_back({&h->kc, cache_bytes, "key cache"});
    bufs.push_back({&h->vtc, cache_bytes, "value cache"});
    bufs.push_back({(void**)&h->x, (size_t)Mp * A * 4, "state rows"});
    bufs.push_back({&h->xb, (size_t)Mp * A * 2, "bf16 state rows"});
    bufs.push_back({(void**)&h->lens, (size_t)c.batch * sizeof(int), "prefix lengths"});
    bufs.push_back({(void**)&h->rope, (size_t)M * (c.head_dim / 2) * sizeof(float2), "position table"});
    bufs.push_back({(void**)&h->part_o, part_rows * c.head_dim * sizeof(float), "attention partials"});
    bufs.push_back({(void**)&h->part_ml, part_rows * sizeof(float2), "attention statistics"});
    // the small-M projections' sums of squares, split partials and counters
    size_t gp = 1;
    for (const GemmPlan* p : {&h->p_in, &h->p_out})
      if (p->KSW > 1) gp = std::max(gp, (size_t)p->NT * p->KSW * h->MT * 256);
    bufs.push_back({(void**)&h->ss, (size_t)h->NTD * h->ss_ld * sizeof(float), "sums of squares"});
    bufs.push_back({(void**)&h->gpart, gp * sizeof(float), "split partials"});
    bufs.push_back({(void**)&h->counters, (size_t)std::max(h->p_in.NT, h->p_out.NT) * sizeof(unsigned),
                    "split counters"});
  } else {
    bufs.push_back({&h->tk, (size_t)(dit ? 1 : NL) * R * kvd * 2, "key rows"});
    bufs.push_back({&h->tv, (size_t)(dit ? 1 : NL) * R * kvd * 2, "value fragments"});
  }
  if (!dit && !h->batched) {
    if (!prefill) {  // the prefill's token rows go straight into the residual rows
      bufs.push_back({(void**)&h->x, (size_t)Mp * A * 4, "state rows"});
      bufs.push_back({&h->xb, (size_t)Mp * A * 2, "bf16 state rows"});
    }
    bufs.push_back({(void**)&h->lens, sizeof(int), "prefix length"});
    bufs.push_back({(void**)&h->rope, (size_t)M * (c.head_dim / 2) * sizeof(float2), "position table"});
  }
  if (h->splits > 1 && !h->batched) {
    bufs.push_back({(void**)&h->po, (size_t)h->splits * M * HD * 4, "attention partials"});
    bufs.push_back({(void**)&h->pml, (size_t)h->splits * M * H * 2 * 4, "attention statistics"});
  }
  for (const Buf& b : bufs) {
    if ((rc = alloc(h, b.p, b.bytes, b.what))) return rc;
    PHX_HIP(hipMemsetAsync(*b.p, 0, b.bytes, stream));
  }
  // the prefill's tokens sit at positions 0 .. M-1 with no cached rows before them
  if (prefill) PHX_HIP(tok::launch_positions(h->lens, h->rope, 0, 0, M, c.head_dim, (double)c.rope_base, stream));
  PHX_HIP(hipStreamSynchronize(stream));
  for (size_t i = 0; etab && i < h->allocs.size(); ++i)
    if (h->allocs[i] == etab) {
      (void)hipFree(etab);
      h->allocs.erase(h->allocs.begin() + (long)i);
      break;
    }

  if (!dit && !prefill && !h->batched) {
    if ((rc = build_tok_nodes(h, true))) return rc;
    h->cnodes.swap(h->tnodes);
  }
  if ((rc = build_tok_nodes(h))) return rc;
  h->nodes = (int)h->tnodes.size();
  size_t part = 0;
  for (const std::vector<TokNode>* list : {&h->tnodes, &h->cnodes})
    for (const TokNode& nd : *list)
      if (nd.op == TOP_GEMM) part = std::max(part, tok::gemm_part_elems(nd.g));
  if (part) {
    if ((rc = alloc(h, (void**)&h->tpart, part * sizeof(float), "GEMM split partials"))) return rc;
    for (std::vector<TokNode>* list : {&h->tnodes, &h->cnodes})
      for (TokNode& nd : *list)
        if (nd.op == TOP_GEMM) nd.g.part = h->tpart;
  }
  PHX_HIP(tok::prepare_gemm());
  PHX_HIP(tok::prepare_attention());
  if (!(c.flags & PHX_FLAG_NO_GRAPH)) {
    if ((rc = capture_tok(h, h->tnodes, &h->graph, &h->exec))) return rc;
    if (!h->cnodes.empty() && (rc = capture_tok(h, h->cnodes, &h->cgraph, &h->cexec))) return rc;
  }
  return PHX_OK;
}


// ---------------------------------------------------------------- capsules
// The declared state regions of a handle: what phx_expert_load_prefix_kv
// writes and every decision reads (the stored prefix K/V, the prefix lengths,
// the decoder position table), in a fixed order per plan.
struct StateRegion {
  const char* name;
  void* ptr;
  size_t bytes;
};

std::vector<StateRegion> state_regions(const phx_expert* h) {
  const phx_expert_config& c = h->cfg;
  std::vector<StateRegion> r;
  if (h->tokens && !h->batched) {
    // the DiT-style step has no prefix, and the prefill hands its cache to the caller:
    // nothing persists between calls
    if (c.block_kind != PHX_BLOCK_DECODER) return r;
    const size_t kv = (size_t)c.layers * h->R * c.n_kv_heads * c.head_dim * 2;
    r.push_back({"key_rows", h->tk, kv});
    r.push_back({"value_fragments", h->tv, kv});
    r.push_back({"prefix_lengths", h->lens, sizeof(int)});
    r.push_back({"position_table", h->rope, (size_t)c.rows * (c.head_dim / 2) * sizeof(float2)});
  } else if (h->persistent) {
    r.push_back({"attention_kv_tiles", h->kvt, (size_t)h->dargs.kvt_bytes});
    r.push_back({"prefix_lengths", h->lens, sizeof(int)});
    r.push_back({"position_table", h->rope, (size_t)c.rows * (c.head_dim / 2) * sizeof(float2)});
  } else {
    const size_t kv = (size_t)c.layers * h->kv_layer * h->esz;
    r.push_back({"key_cache", h->kc, kv});
    r.push_back({"value_cache", h->vtc, kv});
    r.push_back({"prefix_lengths", h->lens, (size_t)c.batch * sizeof(int)});
    r.push_back({"position_table", h->rope, (size_t)c.batch * c.rows * (c.head_dim / 2) * sizeof(float2)});
  }
  return r;
}

constexpr uint32_t CAPSULE_MAGIC = 0x43584850u;  // "PHXC"
constexpr uint32_t CAPSULE_VERSION = 1u;
constexpr int CAPSULE_MAX_REGIONS = 8;

struct CapsuleEntry {
  char name[24];
  uint64_t offset;  // bytes from the start of the capsule
  uint64_t bytes;
};

// Capsule layout: this header, then per request (prefix length, loaded flag,
// position base) as int32 triples, then every region at a 256-byte aligned offset.
struct CapsuleHeader {
  uint32_t magic, version;
  uint64_t fingerprint;  // plan: configuration, execution path, region sizes
  uint64_t total_bytes;
  uint32_t n_regions, batch;
  CapsuleEntry region[CAPSULE_MAX_REGIONS];
};

uint64_t fnv1a(uint64_t h, const void* p, size_t n) {
  const unsigned char* b = (const unsigned char*)p;
  for (size_t i = 0; i < n; ++i) {
    h ^= b[i];
    h *= 1099511628211ull;
  }
  return h;
}

size_t capsule_head_bytes(const phx_expert* h) {
  return align_up(sizeof(CapsuleHeader) + (size_t)h->cfg.batch * 3 * sizeof(int32_t), 256);
}

// header of this handle's capsule (host state included)
CapsuleHeader capsule_layout(const phx_expert* h, const std::vector<StateRegion>& regs) {
  CapsuleHeader hd{};
  hd.magic = CAPSULE_MAGIC;
  hd.version = CAPSULE_VERSION;
  hd.batch = (uint32_t)h->cfg.batch;
  hd.n_regions = (uint32_t)regs.size();
  uint64_t fp = 1469598103934665603ull;
  fp = fnv1a(fp, &h->cfg, sizeof(h->cfg));
  const int path = h->batched ? 3 : h->tokens ? 2 : h->persistent ? 1 : 0;
  fp = fnv1a(fp, &path, sizeof(path));
  size_t off = capsule_head_bytes(h);
  for (size_t i = 0; i < regs.size(); ++i) {
    CapsuleEntry& e = hd.region[i];
    std::snprintf(e.name, sizeof(e.name), "%s", regs[i].name);
    e.offset = off;
    e.bytes = regs[i].bytes;
    fp = fnv1a(fp, &e.bytes, sizeof(e.bytes));
    off = align_up(off + regs[i].bytes, 256);
  }
  hd.total_bytes = off;
  hd.fingerprint = fp;
  return hd;
}

int capsule_staging(phx_expert* h, size_t bytes) {
  if (!h->cap_event) PHX_HIP(hipEventCreateWithFlags(&h->cap_event, hipEventDisableTiming));
  PHX_HIP(hipEventSynchronize(h->cap_event));  // the previous header copy has finished
  if (h->cap_host_bytes < bytes) {
    if (h->cap_host) PHX_HIP(hipHostFree(h->cap_host));
    h->cap_host = nullptr;
    h->cap_host_bytes = 0;
    hipError_t e = hipHostMalloc(&h->cap_host, bytes, hipHostMallocDefault);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      return fail(PHX_E_NOMEM, "pinned capsule staging of %zu bytes failed: %s", bytes, hipGetErrorString(e));
    }
    h->cap_host_bytes = bytes;
  }
  return PHX_OK;
}

}  // namespace

extern "C" {

const char* phx_last_error(void) { return g_err.c_str(); }

int phx_expert_validate_config(const phx_expert_config* c) {
  if (!c) return fail(PHX_E_INVALID, "config is NULL");
  if (c->abi_version != PHX_ABI_VERSION)
    return fail(PHX_E_VERSION, "abi_version %u, library implements %u", c->abi_version, PHX_ABI_VERSION);
  if (c->struct_size != sizeof(phx_expert_config))
    return fail(PHX_E_VERSION, "struct_size %u, library expects %zu", c->struct_size, sizeof(phx_expert_config));
  if (c->layers < 1 || c->layers > 256) return fail(PHX_E_SHAPE, "layers %d outside [1, 256]", c->layers);
  if (c->width < 128 || c->width % 128) return fail(PHX_E_SHAPE, "width %d must be a positive multiple of 128", c->width);
  if (c->head_dim != 64 && c->head_dim != 128 && c->head_dim != 256)
    return fail(PHX_E_SHAPE, "head_dim %d must be 64, 128 or 256", c->head_dim);
  if (c->n_heads < 1 || c->n_kv_heads < 1 || c->n_heads % c->n_kv_heads)
    return fail(PHX_E_SHAPE, "n_kv_heads %d must divide n_heads %d", c->n_kv_heads, c->n_heads);
  if ((c->n_heads * c->head_dim) % 128)
    return fail(PHX_E_SHAPE, "n_heads*head_dim %d must be a multiple of 128", c->n_heads * c->head_dim);
  if (c->mlp_hidden < 128 || c->mlp_hidden % 128)
    return fail(PHX_E_SHAPE, "mlp_hidden %d must be a positive multiple of 128", c->mlp_hidden);
  if (c->state_dim < 32 || c->state_dim % 32)
    return fail(PHX_E_SHAPE, "state_dim %d must be a positive multiple of 32", c->state_dim);
  if (c->block_kind != PHX_BLOCK_DECODER && c->block_kind != PHX_BLOCK_DIT && c->block_kind != PHX_BLOCK_PREFILL)
    return fail(PHX_E_INVALID, "block_kind %d unknown", c->block_kind);
  if (c->mask_kind != PHX_MASK_FULL && c->mask_kind != PHX_MASK_CAUSAL)
    return fail(PHX_E_INVALID, "mask_kind %d unknown", c->mask_kind);
  if ((c->mask_kind == PHX_MASK_CAUSAL) != (c->block_kind == PHX_BLOCK_PREFILL))
    return fail(PHX_E_SHAPE, "the prefix prefill takes the causal mask, the other blocks the full mask");
  if (c->rows < 1 || c->batch < 1) return fail(PHX_E_SHAPE, "rows and batch must be positive");
  const bool tokens = c->block_kind != PHX_BLOCK_DECODER || (long long)c->rows * c->batch > 160;
  if (tokens) {
    // the large-token plan: one chunk of many rows
    if (c->batch != 1 || c->rows > 16384)
      return fail(PHX_E_SHAPE, "the large-token plan needs batch 1 and rows <= 16384 (rows %d, batch %d)", c->rows,
                  c->batch);
    if (c->weight_dtype != PHX_DTYPE_BF16) return fail(PHX_E_SHAPE, "the large-token plan needs bf16 weights");
    if (c->head_dim != 128 && c->head_dim != 256)
      return fail(PHX_E_SHAPE, "the large-token plan needs head_dim 128 or 256");
    if (c->state_dim % 128) return fail(PHX_E_SHAPE, "the large-token plan needs state_dim a multiple of 128");
    if (c->block_kind == PHX_BLOCK_DIT) {
      if (c->state_dim != c->width) return fail(PHX_E_SHAPE, "the DiT-style block needs state_dim == width");
      if (c->n_kv_heads != c->n_heads) return fail(PHX_E_SHAPE, "the DiT-style block needs n_kv_heads == n_heads");
      if (c->prefix_capacity != 0) return fail(PHX_E_SHAPE, "the DiT-style block has no prefix (capacity 0)");
      if (c->steps != 1) return fail(PHX_E_SHAPE, "the DiT-style block runs one step");
    }
    if (c->block_kind == PHX_BLOCK_PREFILL) {
      if (c->state_dim != c->width) return fail(PHX_E_SHAPE, "the prefix prefill needs state_dim == width");
      if (c->prefix_capacity != 0) return fail(PHX_E_SHAPE, "the prefix prefill reads no cache (capacity 0)");
      if (c->steps != 1) return fail(PHX_E_SHAPE, "the prefix prefill runs one pass");
    }
  } else if ((c->n_heads / c->n_kv_heads) * c->rows > 128) {
    return fail(PHX_E_SHAPE, "query rows per kv head (n_heads/n_kv_heads*rows = %d) must be at most 128",
                (c->n_heads / c->n_kv_heads) * c->rows);
  }
  if (c->prefix_capacity < 0 || c->prefix_capacity > 65536)
    return fail(PHX_E_SHAPE, "prefix_capacity %d outside [0, 65536]", c->prefix_capacity);
  if (c->steps < 1 || c->steps > 1000) return fail(PHX_E_SHAPE, "steps %d outside [1, 1000]", c->steps);
  if (c->time_emb_dim < 2 || c->time_emb_dim % 2 || c->time_emb_dim > 65536)
    return fail(PHX_E_SHAPE, "time_emb_dim %d must be even and at most 65536", c->time_emb_dim);
  if (!(c->rms_eps > 0.f) || !std::isfinite(c->rms_eps)) return fail(PHX_E_INVALID, "rms_eps must be positive");
  if (!(c->rope_base > 0.f) || !std::isfinite(c->rope_base)) return fail(PHX_E_INVALID, "rope_base must be positive");
  if (!std::isfinite(c->tau0) || !std::isfinite(c->dt)) return fail(PHX_E_INVALID, "tau0 and dt must be finite");
  if (c->weight_dtype != PHX_DTYPE_F32 && c->weight_dtype != PHX_DTYPE_BF16)
    return fail(PHX_E_INVALID, "weight_dtype %d unknown", c->weight_dtype);
  if (c->kv_dtype != c->weight_dtype) return fail(PHX_E_SHAPE, "kv_dtype must equal weight_dtype");
  if (c->flags & ~(PHX_FLAG_NO_GRAPH | PHX_FLAG_MULTI_KERNEL | PHX_FLAG_TIMELINE | PHX_FLAG_WEIGHTS_INT8 |
                   PHX_FLAG_PAIRED_ACT | PHX_FLAG_BF16_ACT))
    return fail(PHX_E_INVALID, "unknown flags 0x%x", c->flags);
  if ((c->flags & PHX_FLAG_PAIRED_ACT) && (c->flags & PHX_FLAG_BF16_ACT))
    return fail(PHX_E_INVALID, "PHX_FLAG_PAIRED_ACT and PHX_FLAG_BF16_ACT exclude each other");
  if ((c->flags & PHX_FLAG_WEIGHTS_INT8) &&
      (c->weight_dtype != PHX_DTYPE_BF16 || c->block_kind != PHX_BLOCK_DECODER || (long long)c->rows * c->batch > 160))
    return fail(PHX_E_SHAPE, "the 8-bit weight tier needs bf16 weights, the decoder block and at most 160 rows");
  return PHX_OK;
}

int phx_expert_weights_bytes(const phx_expert_config* cfg, size_t* bytes) {
  if (!bytes) return fail(PHX_E_INVALID, "bytes is NULL");
  int rc = phx_expert_validate_config(cfg);
  if (rc) return rc;
  *bytes = weight_elems(cfg) * (cfg->weight_dtype == PHX_DTYPE_BF16 ? 2 : 4);
  return PHX_OK;
}

int phx_expert_weight_codes(const phx_expert* h, int32_t layer, int32_t matrix, int8_t* codes, float* scales,
                            phx_stream_t stream) {
  if (!h || !codes || !scales) return fail(PHX_E_INVALID, "NULL argument");
  if (!h->wq) return fail(PHX_E_STATE, "the handle has no int8 weights (PHX_FLAG_WEIGHTS_INT8)");
  const phx_expert_config& c = h->cfg;
  if (layer < 0 || layer >= c.layers || matrix < 0 || matrix > 3)
    return fail(PHX_E_SHAPE, "layer %d or matrix %d out of range", layer, matrix);
  if (!is_device_pointer(codes) || !is_device_pointer(scales))
    return fail(PHX_E_INVALID, "codes and scales must be device pointers");
  const int D = c.width, HD = c.n_heads * c.head_dim, F = c.mlp_hidden;
  const int qkvN = (c.n_heads + 2 * c.n_kv_heads) * c.head_dim;
  const int K[4] = {D, HD, D, F}, N[4] = {qkvN, D, 2 * F, D};
  const int kind[4] = {COL_ROPE, COL_IDENT, COL_GEGLU, COL_IDENT}, param[4] = {c.head_dim, 0, F, 0};
  const size_t off[4] = {h->off_qkv[layer], h->off_o[layer], h->off_gu[layer], h->off_down[layer]};
  const size_t so[4] = {h->sc_qkv[layer], h->sc_o[layer], h->sc_gu[layer], h->sc_down[layer]};
  PHX_HIP(launch_untile_codes(h->wq + off[matrix], h->wsc + so[matrix], (signed char*)codes, scales, K[matrix],
                              N[matrix], kind[matrix], param[matrix], (hipStream_t)stream));
  g_err.clear();
  return PHX_OK;
}

int phx_expert_kernels_per_decision(const phx_expert* h, int* count) {
  if (!h || !count) return fail(PHX_E_INVALID, "NULL argument");
  *count = h->nodes;
  return PHX_OK;
}

static int create_impl(phx_expert* h, const void* weights, hipStream_t stream) {
  const phx_expert_config& c = h->cfg;
  const int D = c.width, H = c.n_heads, Dh = c.head_dim, KVH = c.n_kv_heads, F = c.mlp_hidden, A = c.state_dim;
  const int M = c.rows, B = c.batch, NL = c.layers, S = c.steps, E = c.time_emb_dim;
  h->dtype = c.weight_dtype == PHX_DTYPE_BF16 ? 1 : 0;
  h->esz = h->dtype ? 2 : 4;
  h->BM = B * M;
  h->MT = mt_for_rows(h->BM);
  h->NTD = D / 16;
  h->ss_ld = 16 * h->MT;
  h->SMAX = (int)((c.prefix_capacity + M + ATTN_KEYS - 1) / ATTN_KEYS);
  h->Ctot = h->SMAX * ATTN_KEYS;
  const int GM = (H / KVH) * M;
  h->QT = (GM + 15) / 16;
  h->GMP = h->QT * 16;
  h->NN = 2 * NL + 1;
  h->kv_layer = (size_t)B * KVH * h->Ctot * Dh;
  const int qkvN = (H + 2 * KVH) * Dh;

  h->p_in = make_plan(A, D, 1);
  // QKV keeps one workgroup per 16-column tile: a k split ends in a store, wait, counter and reload tail
  // that costs more than the extra workgroups gain here (pi0.5 shape: 10.3 -> 9.0 us per launch), while
  // the out and down projections (64 column tiles, K 2048 and 4096) still gain from splitting
  h->p_qkv = make_plan(D, qkvN, 1);
  h->p_o = make_plan(H * Dh, D, 256);
  h->p_gu = make_plan(D, 2 * F, 256);
  h->p_down = make_plan(F, D, 256);
  h->p_out = make_plan(D, A, 256);
  if (h->p_in.NW != 1)  // the input projection kernel runs one wave per workgroup
    h->p_in.NW = 1;

  int rc;
  hipDeviceProp_t prop;
  int dev = 0;
  PHX_HIP(hipGetDevice(&dev));
  h->device = dev;
  PHX_HIP(hipGetDeviceProperties(&prop, dev));
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(PHX_E_HIP, "device %d is %s; this library is built for gfx950 only", dev, prop.gcnArchName);
  PHX_HIP(hipStreamCreateWithFlags(&h->cap, hipStreamNonBlocking));

  // ---- static: tiled weights (everything but W_mod) ----
  // decoder blob: W_in, per layer [W_qkv, W_o, W_gu, W_down], W_out, W_mod;
  // DiT-style blob: per block [W_qkv, W_o, W_up, W_down], W_mod;
  // prefill blob: per layer [W_qkv, W_o, W_gu, W_down], the norm gains
  const bool dit = c.block_kind == PHX_BLOCK_DIT;
  const bool io = c.block_kind == PHX_BLOCK_DECODER;  // in- and out-linears around the stack
  const int gu_cols = dit ? F : 2 * F;
  size_t off = 0;
  h->off_in = off;
  if (io) off += (size_t)A * D;
  for (int l = 0; l < NL; ++l) {
    h->off_qkv.push_back(off); off += (size_t)D * qkvN;
    h->off_o.push_back(off); off += (size_t)H * Dh * D;
    h->off_gu.push_back(off); off += (size_t)D * gu_cols;
    h->off_down.push_back(off); off += (size_t)F * D;
  }
  h->off_out = off;
  if (io) off += (size_t)D * A;
  const size_t tiled_elems = off;
  const size_t total_elems = weight_elems(&c);
  if ((rc = alloc(h, &h->wt, tiled_elems * h->esz, "tiled weights"))) return rc;

  const void* src = weights;
  void* staging = nullptr;
  if (!is_device_pointer(weights)) {
    if ((rc = alloc(h, &staging, total_elems * h->esz, "weight staging"))) return rc;
    PHX_HIP(hipMemcpyAsync(staging, weights, total_elems * h->esz, hipMemcpyHostToDevice, stream));
    src = staging;
  }
  // the blob has the same order as the tiled arena, plus W_mod (the gains of the prefill) at the end
  const char* sb = (const char*)src;
  auto retile = [&](size_t o, int K, int N, int kind, int param) -> int {
    PHX_HIP(launch_retile(h->dtype, sb + o * h->esz, (char*)h->wt + o * h->esz, K, N, kind, param, stream));
    return PHX_OK;
  };
  if (io && (rc = retile(h->off_in, A, D, COL_IDENT, 0))) return rc;
  for (int l = 0; l < NL; ++l) {
    if ((rc = retile(h->off_qkv[l], D, qkvN, COL_ROPE, Dh))) return rc;
    if ((rc = retile(h->off_o[l], H * Dh, D, COL_IDENT, 0))) return rc;
    if ((rc = retile(h->off_gu[l], D, gu_cols, dit ? COL_IDENT : COL_GEGLU, F))) return rc;
    if ((rc = retile(h->off_down[l], F, D, COL_IDENT, 0))) return rc;
  }
  if (io && (rc = retile(h->off_out, D, A, COL_IDENT, 0))) return rc;

  if (c.flags & PHX_FLAG_WEIGHTS_INT8) {
    // the 8-bit tier: codes of every layer's four projections from their tiled bf16 form
    size_t nsc = 0;
    for (int l = 0; l < NL; ++l) {
      h->sc_qkv.push_back(nsc); nsc += (size_t)qkvN;
      h->sc_o.push_back(nsc); nsc += (size_t)D;
      h->sc_gu.push_back(nsc); nsc += (size_t)gu_cols;
      h->sc_down.push_back(nsc); nsc += (size_t)D;
    }
    if ((rc = alloc(h, (void**)&h->wq, tiled_elems, "int8 weight codes"))) return rc;
    if ((rc = alloc(h, (void**)&h->wsc, nsc * sizeof(float), "int8 weight scales"))) return rc;
    auto quant = [&](size_t o, size_t so, int K, int N) -> int {
      PHX_HIP(launch_quant_i8((const char*)h->wt + o * h->esz, h->wq + o, h->wsc + so, K, N, stream));
      return PHX_OK;
    };
    for (int l = 0; l < NL; ++l) {
      if ((rc = quant(h->off_qkv[l], h->sc_qkv[l], D, qkvN))) return rc;
      if ((rc = quant(h->off_o[l], h->sc_o[l], H * Dh, D))) return rc;
      if ((rc = quant(h->off_gu[l], h->sc_gu[l], D, gu_cols))) return rc;
      if ((rc = quant(h->off_down[l], h->sc_down[l], F, D))) return rc;
    }
  }

  h->tokens = uses_tokens(c);
  h->n_cu = prop.multiProcessorCount;
  if (!h->tokens && !persistent_eligible(c, prop) && uses_batched(c)) {
    h->tokens = true;
    h->batched = true;
  }
  if (h->tokens) {
    rc = create_tokens(h, sb, stream, off);
    if (rc) return rc;
    for (size_t i = 0; i < h->allocs.size(); ++i)
      if (staging && h->allocs[i] == staging) {
        (void)hipFree(staging);
        h->allocs.erase(h->allocs.begin() + (long)i);
        break;
      }
    h->loaded.assign(B, dit || c.block_kind == PHX_BLOCK_PREFILL ? 1 : 0);  // no prefix to load
    h->lens_host.assign(B, 0);
    return PHX_OK;
  }

  h->persistent = persistent_eligible(c, prop);
  if (h->persistent) {
    rc = create_persistent(h, sb, stream, off);
    if (rc) return rc;
    for (size_t i = 0; i < h->allocs.size(); ++i)
      if (staging && h->allocs[i] == staging) {
        (void)hipFree(staging);
        h->allocs.erase(h->allocs.begin() + (long)i);
        break;
      }
    h->loaded.assign(B, 0);
    h->lens_host.assign(B, 0);
    return PHX_OK;
  }

  // ---- static: step-conditioning table, built once for the handle's life ----
  void* etab = nullptr;
  if ((rc = alloc(h, &etab, (size_t)S * E * sizeof(double), "time embedding"))) return rc;
  if ((rc = alloc(h, (void**)&h->modtab, (size_t)S * h->NN * 2 * D * sizeof(float), "modulation table"))) return rc;
  PHX_HIP(launch_time_embedding((double*)etab, S, E, c.tau0, c.dt, stream));
  PHX_HIP(launch_modulation(h->dtype, sb + off * h->esz, (const double*)etab, h->modtab, S, h->NN, E, 2 * D, stream));

  // ---- state and working memory ----
  const size_t cache_bytes = (size_t)NL * h->kv_layer * h->esz;
  if ((rc = alloc(h, &h->kc, cache_bytes, "key cache"))) return rc;
  if ((rc = alloc(h, &h->vtc, cache_bytes, "value cache"))) return rc;
  if ((rc = alloc(h, (void**)&h->lens, (size_t)B * sizeof(int), "prefix lengths"))) return rc;
  if ((rc = alloc(h, (void**)&h->rope, (size_t)B * M * (Dh / 2) * sizeof(float2), "position table"))) return rc;
  if ((rc = alloc(h, (void**)&h->x, (size_t)h->BM * A * sizeof(float), "state"))) return rc;
  if ((rc = alloc(h, (void**)&h->h, (size_t)h->BM * D * sizeof(float), "residual stream"))) return rc;
  if ((rc = alloc(h, (void**)&h->ss, (size_t)h->NTD * h->ss_ld * sizeof(float), "sums of squares"))) return rc;
  if ((rc = alloc(h, &h->q, (size_t)h->BM * H * Dh * h->esz, "queries"))) return rc;
  if ((rc = alloc(h, &h->o, (size_t)h->BM * H * Dh * h->esz, "attention output"))) return rc;
  if ((rc = alloc(h, &h->act, (size_t)h->BM * F * h->esz, "GeGLU activation"))) return rc;
  const size_t part_rows = (size_t)B * KVH * h->SMAX * h->GMP;
  if ((rc = alloc(h, (void**)&h->part_o, part_rows * Dh * sizeof(float), "attention partials"))) return rc;
  if ((rc = alloc(h, (void**)&h->part_ml, part_rows * sizeof(float2), "attention statistics"))) return rc;
  size_t gp = 0, maxnt = 0;
  for (const GemmPlan* p : {&h->p_in, &h->p_qkv, &h->p_o, &h->p_gu, &h->p_down, &h->p_out}) {
    if (p->KSW > 1) gp = std::max(gp, (size_t)p->NT * p->KSW * h->MT * 256);
    maxnt = std::max(maxnt, (size_t)p->NT);
  }
  if ((rc = alloc(h, (void**)&h->gpart, std::max(gp, (size_t)1) * sizeof(float), "split partials"))) return rc;
  if ((rc = alloc(h, (void**)&h->counters, maxnt * sizeof(unsigned), "split counters"))) return rc;
  PHX_HIP(hipMemsetAsync(h->kc, 0, cache_bytes, stream));
  PHX_HIP(hipMemsetAsync(h->vtc, 0, cache_bytes, stream));
  PHX_HIP(hipMemsetAsync(h->lens, 0, (size_t)B * sizeof(int), stream));
  PHX_HIP(hipMemsetAsync(h->rope, 0, (size_t)B * M * (Dh / 2) * sizeof(float2), stream));
  PHX_HIP(hipMemsetAsync(h->ss, 0, (size_t)h->NTD * h->ss_ld * sizeof(float), stream));
  PHX_HIP(hipMemsetAsync(h->counters, 0, maxnt * sizeof(unsigned), stream));
  PHX_HIP(hipMemsetAsync(h->x, 0, (size_t)h->BM * A * sizeof(float), stream));
  PHX_HIP(hipMemsetAsync(h->h, 0, (size_t)h->BM * D * sizeof(float), stream));
  PHX_HIP(hipStreamSynchronize(stream));
  // set-up scratch is no longer needed
  for (void* p : {etab, staging}) {
    if (!p) continue;
    for (size_t i = 0; i < h->allocs.size(); ++i)
      if (h->allocs[i] == p) {
        (void)hipFree(p);
        h->allocs.erase(h->allocs.begin() + (long)i);
        break;
      }
  }
  h->loaded.assign(B, 0);
  h->lens_host.assign(B, 0);

  // ---- capture the step loop ----
  if ((rc = build_nodes(h))) return rc;
  h->nodes = (int)h->node_list.size();
  if (!(c.flags & PHX_FLAG_NO_GRAPH)) {
    PHX_HIP(hipStreamBeginCapture(h->cap, hipStreamCaptureModeThreadLocal));
    rc = enqueue_steps(h, h->cap);
    hipGraph_t g = nullptr;
    hipError_t e = hipStreamEndCapture(h->cap, &g);
    if (rc) {
      if (g) (void)hipGraphDestroy(g);
      return rc;
    }
    if (e != hipSuccess) return fail(PHX_E_HIP, "hipStreamEndCapture failed: %s", hipGetErrorString(e));
    h->graph = g;
    PHX_HIP(hipGraphInstantiate(&h->exec, h->graph, nullptr, nullptr, 0));
  }
  return PHX_OK;
}

int phx_expert_create(const phx_expert_config* cfg, const void* weights, size_t weights_bytes, phx_stream_t stream,
                      phx_expert** out) {
  if (!out) return fail(PHX_E_INVALID, "out is NULL");
  int rc = phx_expert_validate_config(cfg);
  if (rc) return rc;
  if (!weights) return fail(PHX_E_INVALID, "weights is NULL");
  const size_t want = weight_elems(cfg) * (cfg->weight_dtype == PHX_DTYPE_BF16 ? 2 : 4);
  if (weights_bytes != want) return fail(PHX_E_SHAPE, "weights_bytes %zu, expected %zu", weights_bytes, want);
  phx_expert* h = new (std::nothrow) phx_expert();
  if (!h) return fail(PHX_E_NOMEM, "host allocation failed");
  h->cfg = *cfg;
  rc = create_impl(h, weights, (hipStream_t)stream);
  if (rc) {
    std::string msg = g_err;
    release(h);
    g_err = msg;
    return rc;
  }
  *out = h;
  g_err.clear();
  return PHX_OK;
}

int phx_expert_load_prefix_kv(phx_expert* h, int32_t request, const void* k, const void* v, int32_t prefix_len,
                              phx_stream_t stream) {
  if (!h) return fail(PHX_E_INVALID, "handle is NULL");
  const phx_expert_config& c = h->cfg;
  if (request < 0 || request >= c.batch) return fail(PHX_E_SHAPE, "request %d outside [0, %d)", request, c.batch);
  if (prefix_len < 0 || prefix_len > c.prefix_capacity)
    return fail(PHX_E_SHAPE, "prefix_len %d outside [0, %d]", prefix_len, c.prefix_capacity);
  if (prefix_len > 0 && (!k || !v)) return fail(PHX_E_INVALID, "k or v is NULL");
  if (prefix_len > 0 && (!is_device_pointer(k) || !is_device_pointer(v)))
    return fail(PHX_E_INVALID, "k and v must be device pointers");
  hipStream_t s = (hipStream_t)stream;
  if (c.block_kind == PHX_BLOCK_PREFILL)
    return fail(PHX_E_INVALID, "a prefix prefill handle reads no prefix (it writes one: phx_expert_prefill)");
  if (h->tokens && c.block_kind == PHX_BLOCK_DIT) {
    h->loaded[request] = 1;  // capacity 0: nothing to copy
    g_err.clear();
    return PHX_OK;
  }
  if (h->tokens && !h->batched) {
    // keys [NL][L][kvd] -> rows 0..L-1 of each layer's key rows (rows from L on are the chunk's, or
    // masked); values into the fragment order, zeros from key L on
    const size_t row = (size_t)c.n_kv_heads * c.head_dim * 2;
    if (prefix_len > 0)
      PHX_HIP(hipMemcpy2DAsync(h->tk, (size_t)h->R * row, k, (size_t)prefix_len * row, (size_t)prefix_len * row,
                               (size_t)c.layers, hipMemcpyDeviceToDevice, s));
    PHX_HIP(tok::launch_vt_load(v, h->tv, c.layers, prefix_len, h->R, c.n_kv_heads, c.head_dim, s));
  } else if (h->persistent) {
    PHX_HIP(dec::launch_attn_tiles(k, v, h->kvt, c.layers, prefix_len, h->n_chunks, s));
  } else {
    PHX_HIP(launch_load_prefix(h->dtype, k, v, h->kc, h->vtc, c.layers, c.batch, c.n_kv_heads, c.head_dim, h->Ctot,
                               request, prefix_len, s));
  }
  PHX_HIP(launch_position_table(h->lens, h->rope, request, prefix_len, c.rows, c.head_dim, (double)c.rope_base, s));
  h->loaded[request] = 1;
  h->lens_host[request] = prefix_len;
  if (request == 0) h->pos_base = 0;  // a new context starts at position 0
  g_err.clear();
  return PHX_OK;
}

int phx_expert_commit_chunk(phx_expert* h, const float* chunk, phx_stream_t stream) {
  if (!h || !chunk) return fail(PHX_E_INVALID, "NULL argument");
  if (!h->tokens || h->batched || h->cfg.block_kind != PHX_BLOCK_DECODER || h->cnodes.empty())
    return fail(PHX_E_SHAPE, "commit needs the large-token decoder plan (one request of more than 160 rows)");
  if (!h->loaded[0]) return fail(PHX_E_STATE, "request 0 has no prefix loaded");
  const phx_expert_config& c = h->cfg;
  const int M = c.rows, C = c.prefix_capacity, NL = c.layers;
  if (M > C) return fail(PHX_E_SHAPE, "a chunk of %d rows does not fit a window of %d rows", M, C);
  hipStream_t s = (hipStream_t)stream;
  // the chunk becomes the state rows; one pass writes its keys and values after the L cached rows
  PHX_HIP(hipMemcpyAsync(h->x, chunk, (size_t)M * c.state_dim * sizeof(float), hipMemcpyDefault, s));
  if (h->cexec) {
    PHX_HIP(hipGraphLaunch(h->cexec, s));
  } else {
    for (const TokNode& nd : h->cnodes) {
      int rc = launch_tok(h, nd, s);
      if (rc) return rc;
    }
  }
  int L = h->lens_host[0] + M;
  int base = h->pos_base;
  if (L > C) {
    // window: drop the d oldest rows; the kept keys keep their positions (base + row)
    const int d = L - C;
    const size_t row = (size_t)c.n_kv_heads * c.head_dim * 2;
    const size_t kv = (size_t)NL * h->R * row;
    if (!h->tk_tmp && alloc(h, &h->tk_tmp, kv, "history key staging")) return PHX_E_NOMEM;
    if (!h->tv_tmp && alloc(h, &h->tv_tmp, kv, "history value staging")) return PHX_E_NOMEM;
    PHX_HIP(hipMemcpy2DAsync(h->tk_tmp, (size_t)h->R * row, (const char*)h->tk + (size_t)d * row, (size_t)h->R * row,
                             (size_t)C * row, (size_t)NL, hipMemcpyDeviceToDevice, s));
    PHX_HIP(hipMemcpyAsync(h->tk, h->tk_tmp, kv, hipMemcpyDeviceToDevice, s));
    PHX_HIP(tok::launch_vt_shift(h->tv, h->tv_tmp, NL, c.n_kv_heads, h->R, d, L, c.head_dim, s));
    PHX_HIP(hipMemcpyAsync(h->tv, h->tv_tmp, kv, hipMemcpyDeviceToDevice, s));
    L = C;
    base += d;
  }
  // the next chunk's rows sit after the history
  PHX_HIP(tok::launch_positions(h->lens, h->rope, L, base + L, M, c.head_dim, (double)c.rope_base, s));
  h->lens_host[0] = L;
  h->pos_base = base;
  g_err.clear();
  return PHX_OK;
}

int phx_expert_decide(phx_expert* h, const float* noise, float* actions, phx_stream_t stream) {
  if (!h) return fail(PHX_E_INVALID, "handle is NULL");
  if (!noise || !actions) return fail(PHX_E_INVALID, "noise or actions is NULL");
  if (h->cfg.block_kind == PHX_BLOCK_PREFILL)
    return fail(PHX_E_INVALID, "a prefix prefill handle makes no decision (phx_expert_prefill)");
  for (int b = 0; b < h->cfg.batch; ++b)
    if (!h->loaded[b]) return fail(PHX_E_STATE, "request %d has no prefix loaded", b);
  hipStream_t s = (hipStream_t)stream;
  const size_t xb = (size_t)h->BM * h->cfg.state_dim * sizeof(float);
  // the DiT-style block integrates nothing: its state is the residual stream itself
  float* state = (h->tokens && h->cfg.block_kind == PHX_BLOCK_DIT) ? h->h : h->x;
  PHX_HIP(hipMemcpyAsync(state, noise, xb, hipMemcpyDefault, s));
  if (h->exec) {
    PHX_HIP(hipGraphLaunch(h->exec, s));
  } else {
    int rc = enqueue_steps(h, s);
    if (rc) return rc;
  }
  PHX_HIP(hipMemcpyAsync(actions, state, xb, hipMemcpyDefault, s));
  g_err.clear();
  return PHX_OK;
}

// The decision of phx_expert_decide with the exchange and control words in the
// device's static scratch instead of the handle's arena: stream-ordered
// copies and three kernel launches (prepare, decision, advance), nothing
// allocated, no runtime call that allocates.  Every such call on one device
// shares that scratch; the prepare kernel clears it when the previous
// decision on it had another shape.
int phx_expert_decide_noalloc(phx_expert* h, const float* noise, float* actions, phx_stream_t stream) {
  if (!h) return fail(PHX_E_INVALID, "handle is NULL");
  if (!noise || !actions) return fail(PHX_E_INVALID, "noise or actions is NULL");
  if (!h->persistent)
    return fail(PHX_E_SHAPE,
                "no allocation-free decision for this handle: its plan's working memory is not the decision "
                "kernel's %u bytes of exchange words (the most the static scratch holds); use phx_expert_decide",
                dec::SCRATCH_BYTES);
  if (dec::XC_BYTES > dec::SCRATCH_BYTES)
    return fail(PHX_E_SHAPE, "exchange words of %u bytes exceed the static scratch of %u bytes", dec::XC_BYTES,
                dec::SCRATCH_BYTES);
  if (!h->loaded[0]) return fail(PHX_E_STATE, "request 0 has no prefix loaded");
  if (h->scratch_rc != hipSuccess)
    return fail(PHX_E_HIP, "static scratch of device %d not set up: %s", h->device, hipGetErrorString(h->scratch_rc));
  void* ex = nullptr;
  if (dec::decide_scratch(h->device, &ex) != hipSuccess || !ex)
    return fail(PHX_E_HIP, "static scratch of device %d not set up", h->device);
  hipStream_t s = (hipStream_t)stream;
  const size_t xb = (size_t)h->BM * h->cfg.state_dim * sizeof(float);
  dec::Args a = h->dargs;
  a.ex = ex;
  PHX_HIP(hipMemcpyAsync(h->x, noise, xb, hipMemcpyDefault, s));
  PHX_HIP(dec::launch_decide_prepare(a, s));
  PHX_HIP(dec::launch_decide(a, s));
  PHX_HIP(dec::launch_decide_advance(a, s));
  PHX_HIP(hipMemcpyAsync(actions, h->x, xb, hipMemcpyDefault, s));
  g_err.clear();
  return PHX_OK;
}

int phx_expert_prefill(phx_expert* h, const float* x, int32_t prefix_len, void* k, void* v, phx_stream_t stream) {
  if (!h) return fail(PHX_E_INVALID, "handle is NULL");
  const phx_expert_config& c = h->cfg;
  if (c.block_kind != PHX_BLOCK_PREFILL) return fail(PHX_E_INVALID, "not a prefix prefill handle");
  if (prefix_len < 0 || prefix_len > c.rows)
    return fail(PHX_E_SHAPE, "prefix_len %d outside [0, %d]", prefix_len, c.rows);
  if (prefix_len == 0) {
    g_err.clear();
    return PHX_OK;
  }
  if (!x || !k || !v) return fail(PHX_E_INVALID, "x, k or v is NULL");
  if (!is_device_pointer(k) || !is_device_pointer(v)) return fail(PHX_E_INVALID, "k and v must be device pointers");
  hipStream_t s = (hipStream_t)stream;
  // the tokens become the residual rows; rows past the prefix are zeros (finite, and under the
  // causal mask no earlier row sees them)
  const size_t xrow = (size_t)c.width * sizeof(float);
  PHX_HIP(hipMemcpyAsync(h->h, x, (size_t)prefix_len * xrow, hipMemcpyDefault, s));
  if (prefix_len < c.rows)
    PHX_HIP(hipMemsetAsync((char*)h->h + (size_t)prefix_len * xrow, 0, (size_t)(c.rows - prefix_len) * xrow, s));
  if (h->exec) {
    PHX_HIP(hipGraphLaunch(h->exec, s));
  } else {
    for (const TokNode& nd : h->tnodes) {
      int rc = launch_tok(h, nd, s);
      if (rc) return rc;
    }
  }
  // every layer's keys (rows) and values (fragment order) of the first prefix_len tokens
  const size_t kvrow = (size_t)c.n_kv_heads * c.head_dim * 2;
  PHX_HIP(hipMemcpy2DAsync(k, (size_t)prefix_len * kvrow, h->tk, (size_t)h->R * kvrow, (size_t)prefix_len * kvrow,
                           (size_t)c.layers, hipMemcpyDeviceToDevice, s));
  PHX_HIP(tok::launch_vt_export(h->tv, v, c.layers, prefix_len, h->R, c.n_kv_heads, c.head_dim, s));
  g_err.clear();
  return PHX_OK;
}

int phx_expert_node_info(const phx_expert* h, int32_t node, phx_node_info* info) {
  if (!h || !info) return fail(PHX_E_INVALID, "NULL argument");
  if (node < 0 || node >= h->nodes) return fail(PHX_E_SHAPE, "node %d outside [0, %d)", node, h->nodes);
  std::memset(info, 0, sizeof(*info));
  if (h->tokens) {
    const TokNode& tn = h->tnodes[(size_t)node];
    info->kind = tn.kind;
    info->step = tn.step;
    info->layer = tn.layer;
    info->bytes = tn.bytes;
    if (tn.kind == PHX_NODE_ATTENTION) {
      // query rows, the valid prefix keys and values, the rows' own key and value rows, the output
      const phx_expert_config& c = h->cfg;
      const uint64_t kvd = (uint64_t)c.n_kv_heads * c.head_dim, hd = (uint64_t)c.n_heads * c.head_dim;
      uint64_t bytes = 0;
      for (int b = 0; b < c.batch; ++b)
        bytes += 2 * ((uint64_t)h->lens_host[(size_t)b] * kvd * 2 + (uint64_t)c.rows * (hd + kvd) * 2);
      info->bytes = bytes;
    }
    std::snprintf(info->name, sizeof(info->name), "%s", tn.name);
    return PHX_OK;
  }
  const Node& nd = h->node_list[(size_t)node];
  info->kind = nd.kind;
  info->step = nd.step;
  info->layer = nd.layer;
  info->bytes = nd.bytes;
  if (nd.kind == PHX_NODE_DECISION) {
    // every weight matrix of the step loop, the valid prefix K/V and the
    // modulation rows, once per Euler step; on the 8-bit tier a layer
    // projection is one byte per code plus a float scale per output column
    const phx_expert_config& c = h->cfg;
    const uint64_t D = (uint64_t)c.width, F = (uint64_t)c.mlp_hidden, A = (uint64_t)c.state_dim;
    const uint64_t qkv = (uint64_t)(c.n_heads + 2 * c.n_kv_heads) * c.head_dim, hd = (uint64_t)c.n_heads * c.head_dim;
    const uint64_t proj = D * qkv + hd * D + D * 2 * F + F * D;
    const uint64_t w_layer = h->wq ? proj + sizeof(float) * (qkv + D + 2 * F + D) : proj * h->esz;
    const uint64_t w = (uint64_t)c.layers * w_layer + 2 * A * D * h->esz;
    uint64_t kv = 0;
    for (int b = 0; b < c.batch; ++b)
      kv += 2ull * c.layers * (uint64_t)h->lens_host[(size_t)b] * c.n_kv_heads * c.head_dim * h->esz;
    const uint64_t mod = (uint64_t)(2 * c.layers + 1) * 2 * D * sizeof(float);
    info->bytes = (uint64_t)c.steps * (w + kv + mod);
  }
  if (nd.kind == PHX_NODE_ATTENTION) {
    // valid prefix rows plus the action rows, keys and values, of every request
    const phx_expert_config& c = h->cfg;
    uint64_t rows = 0;
    for (int b = 0; b < c.batch; ++b) rows += (uint64_t)h->lens_host[(size_t)b] + (uint64_t)c.rows;
    info->bytes = 2 * rows * (uint64_t)c.n_kv_heads * c.head_dim * h->esz;
  }
  std::snprintf(info->name, sizeof(info->name), "%s", nd.name);
  return PHX_OK;
}

int phx_expert_launch_node(phx_expert* h, int32_t node, phx_stream_t stream) {
  if (!h) return fail(PHX_E_INVALID, "handle is NULL");
  if (node < 0 || node >= h->nodes) return fail(PHX_E_SHAPE, "node %d outside [0, %d)", node, h->nodes);
  for (int b = 0; b < h->cfg.batch; ++b)
    if (!h->loaded[(size_t)b]) return fail(PHX_E_STATE, "request %d has no prefix loaded", b);
  int rc;
  if (h->persistent && node == 0) {
    rc = enqueue_persistent(h, (hipStream_t)stream);  // the kernel and its tag advance
    if (rc) return rc;
  } else if (h->persistent) {
    // the counter advance belongs to the decision kernel it follows (its use counters run without a gap
    // from one decision to the next), so the diagnostic launch of this node alone does nothing
    (void)stream;
  } else if (h->tokens) {
    rc = launch_tok(h, h->tnodes[(size_t)node], (hipStream_t)stream);
    if (rc) return rc;
  } else {
    rc = launch_node(h, h->node_list[(size_t)node], (hipStream_t)stream);
    if (rc) return rc;
  }
  g_err.clear();
  return PHX_OK;
}

int phx_expert_status(const phx_expert* h, uint32_t* status) {
  if (!h || !status) return fail(PHX_E_INVALID, "NULL argument");
  *status = 0;
  if (!h->persistent) return PHX_OK;
  uint32_t w = 0;  // set after each decision: 1 if a wait of it gave up
  PHX_HIP(hipMemcpy(&w, (const char*)h->arena + dec::AUX0 + dec::AUX_FAILED, sizeof(uint32_t),
                    hipMemcpyDeviceToHost));
  *status = w != 0 ? 1u : 0u;
  return PHX_OK;
}

int phx_expert_timeline(const phx_expert* h, uint32_t* out, size_t capacity, size_t* count) {
  if (!h || !count) return fail(PHX_E_INVALID, "NULL argument");
  *count = 0;
  if (!h->persistent || h->dargs.tl == 0) return fail(PHX_E_STATE, "no timeline: create the handle with PHX_FLAG_TIMELINE");
  const size_t n = (size_t)dec::G * dec::timeline_events(h->cfg.steps, h->cfg.layers);
  if (!out || capacity < n) {
    *count = n;
    return fail(PHX_E_SHAPE, "timeline needs %zu words", n);
  }
  PHX_HIP(hipMemcpy(out, (const char*)h->arena + dec::AUX0 + dec::aux_timeline(h->cfg.steps, h->cfg.layers),
                    n * sizeof(uint32_t), hipMemcpyDeviceToHost));
  *count = n;
  return PHX_OK;
}

int phx_expert_capsule_bytes(const phx_expert* h, size_t* bytes) {
  if (!h || !bytes) return fail(PHX_E_INVALID, "NULL argument");
  *bytes = capsule_layout(h, state_regions(h)).total_bytes;
  g_err.clear();
  return PHX_OK;
}

int phx_expert_capsule_regions(const phx_expert* h, phx_capsule_region* out, int32_t capacity, int32_t* count) {
  if (!h || !count) return fail(PHX_E_INVALID, "NULL argument");
  const std::vector<StateRegion> regs = state_regions(h);
  const CapsuleHeader hd = capsule_layout(h, regs);
  *count = (int32_t)regs.size();
  if (out && capacity < (int32_t)regs.size()) return fail(PHX_E_SHAPE, "capsule has %zu regions", regs.size());
  for (size_t i = 0; out && i < regs.size(); ++i) {
    std::memset(&out[i], 0, sizeof(out[i]));
    std::snprintf(out[i].name, sizeof(out[i].name), "%s", hd.region[i].name);
    out[i].offset = hd.region[i].offset;
    out[i].bytes = hd.region[i].bytes;
  }
  g_err.clear();
  return PHX_OK;
}

int phx_expert_capsule_save(phx_expert* h, void* capsule, size_t bytes, phx_stream_t stream) {
  if (!h || !capsule) return fail(PHX_E_INVALID, "NULL argument");
  const std::vector<StateRegion> regs = state_regions(h);
  const CapsuleHeader hd = capsule_layout(h, regs);
  if (bytes < hd.total_bytes) return fail(PHX_E_SHAPE, "capsule of %zu bytes, needs %llu", bytes,
                                          (unsigned long long)hd.total_bytes);
  if (!is_device_pointer(capsule)) return fail(PHX_E_INVALID, "the capsule must be device memory");
  hipStream_t s = (hipStream_t)stream;
  const size_t head = capsule_head_bytes(h);
  int rc = capsule_staging(h, head);
  if (rc) return rc;
  unsigned char* st = (unsigned char*)h->cap_host;
  std::memset(st, 0, head);
  std::memcpy(st, &hd, sizeof(hd));
  int32_t* hs = (int32_t*)(st + sizeof(CapsuleHeader));
  for (int b = 0; b < h->cfg.batch; ++b) {
    hs[3 * b] = h->lens_host[(size_t)b];
    hs[3 * b + 1] = h->loaded[(size_t)b];
    hs[3 * b + 2] = b == 0 ? h->pos_base : 0;
  }
  PHX_HIP(hipMemcpyAsync(capsule, st, head, hipMemcpyHostToDevice, s));
  PHX_HIP(hipEventRecord(h->cap_event, s));
  for (size_t i = 0; i < regs.size(); ++i)
    PHX_HIP(hipMemcpyAsync((char*)capsule + hd.region[i].offset, regs[i].ptr, regs[i].bytes, hipMemcpyDeviceToDevice,
                           s));
  g_err.clear();
  return PHX_OK;
}

int phx_expert_capsule_restore(phx_expert* h, const void* capsule, size_t bytes, phx_stream_t stream) {
  if (!h || !capsule) return fail(PHX_E_INVALID, "NULL argument");
  const std::vector<StateRegion> regs = state_regions(h);
  const CapsuleHeader want = capsule_layout(h, regs);
  if (bytes < want.total_bytes) return fail(PHX_E_SHAPE, "capsule of %zu bytes, needs %llu", bytes,
                                            (unsigned long long)want.total_bytes);
  if (!is_device_pointer(capsule)) return fail(PHX_E_INVALID, "the capsule must be device memory");
  hipStream_t s = (hipStream_t)stream;
  const size_t head = capsule_head_bytes(h);
  int rc = capsule_staging(h, head);
  if (rc) return rc;
  // the header is needed on the host: read it in stream order and wait for it
  PHX_HIP(hipMemcpyAsync(h->cap_host, capsule, head, hipMemcpyDeviceToHost, s));
  PHX_HIP(hipStreamSynchronize(s));
  CapsuleHeader hd;
  std::memcpy(&hd, h->cap_host, sizeof(hd));
  if (hd.magic != CAPSULE_MAGIC || hd.version != CAPSULE_VERSION)
    return fail(PHX_E_INVALID, "not a capsule of this library (magic 0x%08x, version %u)", hd.magic, hd.version);
  if (hd.fingerprint != want.fingerprint || hd.n_regions != want.n_regions || hd.total_bytes != want.total_bytes)
    return fail(PHX_E_SHAPE, "capsule plan fingerprint %016llx does not match this handle's %016llx",
                (unsigned long long)hd.fingerprint, (unsigned long long)want.fingerprint);
  for (size_t i = 0; i < regs.size(); ++i)
    PHX_HIP(hipMemcpyAsync(regs[i].ptr, (const char*)capsule + hd.region[i].offset, regs[i].bytes,
                           hipMemcpyDeviceToDevice, s));
  const int32_t* hs = (const int32_t*)((const unsigned char*)h->cap_host + sizeof(CapsuleHeader));
  for (int b = 0; b < h->cfg.batch; ++b) {
    h->lens_host[(size_t)b] = hs[3 * b];
    h->loaded[(size_t)b] = hs[3 * b + 1];
  }
  h->pos_base = hs[2];
  g_err.clear();
  return PHX_OK;
}

void phx_expert_destroy(phx_expert* h) { release(h); }

}  // extern "C"
