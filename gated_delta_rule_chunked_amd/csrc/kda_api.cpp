// kda_api.cpp -- the C ABI declared in include/kda.h: host-side validation,
// workspace sizing and kernel launches on the caller's stream.  No allocation,
// no synchronisation, no state kept between calls.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>

#include "../../include/kda.h"
#include "kda_device.hpp"
#include "kda_internal.hpp"
#include "kda_plan.hpp"

static_assert(offsetof(kda_fwd_args, scale) == 40 && offsetof(kda_fwd_args, B) == 64 &&
                  offsetof(kda_fwd_args, o) == 96 && offsetof(kda_fwd_args, stream) == 128 &&
                  offsetof(kda_fwd_args, flags) == 136 && offsetof(kda_fwd_args, hc) == 144 &&
                  offsetof(kda_fwd_args, seg_chunks) == 152 && offsetof(kda_fwd_args, chunk) == 156 &&
                  sizeof(kda_fwd_args) == 160,
              "argument struct layout (mirrored by the Python binding)");
static_assert(offsetof(kda_bwd_dhu_args, scale) == 56 && offsetof(kda_bwd_dhu_args, B) == 72 &&
                  offsetof(kda_bwd_dhu_args, dv2) == 96 && offsetof(kda_bwd_dhu_args, stream) == 136 &&
                  offsetof(kda_bwd_dhu_args, flags) == 144 && offsetof(kda_bwd_dhu_args, seg_chunks) == 148 &&
                  sizeof(kda_bwd_dhu_args) == 152,
              "backward argument struct layout (mirrored by the Python binding)");
static_assert(kda::FLAG_BETA_LOGITS == KDA_FLAG_BETA_LOGITS && kda::FLAG_STATE_BF16 == KDA_FLAG_STATE_BF16 &&
                  kda::FLAG_CKPT_BF16 == KDA_FLAG_CKPT_BF16,
              "flag bits match the public header");

// Scratch of kda_fwd_no_alloc: one static array per device the library runs on, held
// until the process ends.  In host code `scratch` names a host-side stand-in, not a
// device address: kernels and copies get the address looked up by
// hipGetSymbolAddress on the device in question (scratch_on_current_device).
static __device__ __attribute__((aligned(256))) uint8_t scratch[KDA_NO_ALLOC_MAX_BYTES];

namespace {

thread_local char g_hip_msg[256] = "no HIP error recorded";

bool aligned(const void* ptr, uintptr_t a) { return ((uintptr_t)ptr % a) == 0; }

int64_t rec_bytes(int K) { return K == 128 ? kda::Rec<128>::BYTES : kda::Rec<64>::BYTES; }

int64_t round256(int64_t x) { return (x + 255) / 256 * 256; }

// Shape checks shared by every entry point.  Fills the layout on success.
//
// Choice of scan (kda_inter.hip or kda_scan.hip): kda_plan.hpp.  A positive
// seg_chunks selects kda_scan.hip with that segment length.
int check_shapes(const kda_fwd_args* a, kda::WsLayout* L) {
  if (!a) return KDA_ERR_INVALID_ARG;
  if (a->K != 64 && a->K != 128) return KDA_ERR_UNSUPPORTED;
  if (a->V <= 0 || a->V % kda::BV != 0) return KDA_ERR_UNSUPPORTED;
  if (a->B < 1 || a->T < 0 || a->HQK < 1 || a->HV < 1 || a->N < 1) return KDA_ERR_INVALID_ARG;
  if (a->HV % a->HQK != 0) return KDA_ERR_INVALID_ARG;
  if (a->seg_chunks < 0) return KDA_ERR_INVALID_ARG;
  if (a->chunk != 0 && a->chunk != 64 && a->chunk != 16) return KDA_ERR_UNSUPPORTED;
  if (a->cu_seqlens) {
    if (a->B != 1) return KDA_ERR_INVALID_ARG;
  } else if (a->N != a->B) {
    return KDA_ERR_INVALID_ARG;
  }
  // every element index must fit in int64 and every grid in int32
  const int64_t rows = (int64_t)a->B * a->T;
  if (rows > ((int64_t)1 << 40)) return KDA_ERR_INVALID_ARG;
  const int64_t nt = ((int64_t)a->T + kda::BT - 1) / kda::BT;
  const int64_t max_chunks = a->cu_seqlens ? nt + a->N : (int64_t)a->B * nt;
  if (max_chunks * a->HV >= ((int64_t)1 << 31) - 8) return KDA_ERR_INVALID_ARG;
  const int64_t units16 = (int64_t)a->N * a->HV * (a->V / kda::BV);
  if (units16 >= ((int64_t)1 << 31) - 8) return KDA_ERR_INVALID_ARG;
  if (a->N >= (1 << 30)) return KDA_ERR_INVALID_ARG;
  // scan choice and segment plan
  kda::ScanPlan plan = kda::choose_scan(nt, a->cu_seqlens != nullptr, a->N, a->HV, a->V,
                                        a->seg_chunks > 0 ? 0 : kda::device_cus(), a->seg_chunks);
  // chunk 16 runs on the 64-column scan only: where the serial scan would be chosen,
  // one segment per sequence
  if (a->chunk == 16 && !plan.seg_path) plan = {true, std::max<int64_t>(nt, 1)};
  const bool seg_path = plan.seg_path;
  int64_t seg_L = plan.seg_L;
  seg_L = std::min<int64_t>(seg_L, std::max<int64_t>(nt, 1));
  int64_t seg_S = 1, max_segs = 0;
  bool multi = false;
  if (seg_path) {
    if (a->cu_seqlens) {
      // sum over sequences of max(1, ceil(nc / L)) <= chunks / L + N, chunks <= nt + N
      max_segs = (nt + a->N) / seg_L + a->N;
      multi = seg_L < nt;
    } else {
      seg_S = std::max<int64_t>(1, (nt + seg_L - 1) / seg_L);
      max_segs = (int64_t)a->B * seg_S;
      multi = seg_S > 1;
    }
    if (max_segs * a->HV * ((a->V + 63) / 64 + a->K / 64) >= ((int64_t)1 << 31) - 8) return KDA_ERR_INVALID_ARG;
  }
  L->seg_path = seg_path;
  L->seg_L = (int)seg_L;
  L->seg_S = (int)seg_S;
  L->max_segs = max_segs;
  L->rec_bytes = rec_bytes(a->K);
  L->max_chunks = max_chunks;
  const int64_t recs = max_chunks * a->HV * L->rec_bytes;
  // header: counter | varlen: chunk table (N + 2) | segment table (N + 1, segmented scan) | chunk info
  L->cinfo_off = 0;
  L->order_off = 0;
  int64_t head = 16;
  if (a->cu_seqlens) {
    head += ((int64_t)a->N + 2) * 4 + (seg_path ? ((int64_t)a->N + 1) * 4 : 0);
    if (!multi && a->N <= kda::ORDER_MAX_N) {   // one scan per (sequence, head, tile): longest first
      L->order_off = head;
      head += (int64_t)a->N * 4;
    }
    L->cinfo_off = (head + 7) / 8 * 8;
    head = L->cinfo_off + max_chunks * 8;
  }
  L->table_bytes = recs == 0 ? 0 : round256(head);
  const int64_t bbytes = multi ? max_segs * a->HV * a->K * a->V * 4 : 0;
  const int64_t mbytes = multi ? max_segs * a->HV * a->K * a->K * 2 : 0;
  // the segmented scan copies records in whole KiB: 1 KiB of slack after the last
  L->b_off = recs == 0 ? 0 : round256(L->table_bytes + recs + (seg_path ? 1024 : 0));
  L->m_off = L->b_off + bbytes;
  L->total_bytes = L->m_off + mbytes;
  return KDA_OK;
}

enum Need { NEED_INTRA = 1, NEED_INTER = 2 };

// Everything a call needs but its workspace: shapes, tensor pointers and their
// alignment, options, the scale.
int check_args(const kda_fwd_args* a, int need, kda::WsLayout* L) {
  int st = check_shapes(a, L);
  if (st != KDA_OK) return st;
  const bool any_tokens = (int64_t)a->B * a->T > 0;
  if (need & NEED_INTRA) {
    if (any_tokens && (!a->q || !a->k || !a->g || !a->beta)) return KDA_ERR_INVALID_ARG;
    if (!aligned(a->q, 16) || !aligned(a->k, 16) || !aligned(a->g, 16) || !aligned(a->beta, 2))
      return KDA_ERR_INVALID_ARG;
  }
  if (need & NEED_INTER) {
    if (any_tokens && (!a->v || !a->o)) return KDA_ERR_INVALID_ARG;
    if (!aligned(a->v, 16) || !aligned(a->o, 8) || !aligned(a->h0, 16) || !aligned(a->ht, 16))
      return KDA_ERR_INVALID_ARG;
  }
  if (!aligned(a->cu_seqlens, 8) || !aligned(a->hc, 16)) return KDA_ERR_INVALID_ARG;
  if (a->chunk == 16 && a->hc) return KDA_ERR_UNSUPPORTED;
  if (a->flags & ~(uint32_t)(KDA_FLAG_BETA_LOGITS | KDA_FLAG_STATE_BF16)) return KDA_ERR_INVALID_ARG;
  if (!(a->scale == a->scale)) return KDA_ERR_INVALID_ARG;  // NaN scale
  return KDA_OK;
}

int check_call(const kda_fwd_args* a, int need, kda::Params* p) {
  kda::WsLayout L;
  int st = check_args(a, need, &L);
  if (st != KDA_OK) return st;
  if (L.total_bytes > 0) {
    if (!a->workspace || !aligned(a->workspace, 256)) return KDA_ERR_WORKSPACE;
    if (a->workspace_bytes < (size_t)L.total_bytes) return KDA_ERR_WORKSPACE;
  }
  p->q = (const uint16_t*)a->q;
  p->k = (const uint16_t*)a->k;
  p->v = (const uint16_t*)a->v;
  p->g = (const uint16_t*)a->g;
  p->beta = (const uint16_t*)a->beta;
  p->h0 = a->h0;
  p->cu = a->cu_seqlens;
  p->o = (uint16_t*)a->o;
  p->ht = a->ht;
  p->hc = a->hc;
  p->flags = a->flags;
  p->c16 = a->chunk == 16;
  uint8_t* ws = (uint8_t*)a->workspace;
  p->counter = (int32_t*)ws;
  p->table = a->cu_seqlens ? (int32_t*)(ws + 16) : nullptr;
  p->segtab = (a->cu_seqlens && L.seg_path) ? (int32_t*)(ws + 16 + ((int64_t)a->N + 2) * 4) : nullptr;
  p->cinfo = a->cu_seqlens ? (int2*)(ws + L.cinfo_off) : nullptr;
  p->order = L.order_off ? (int32_t*)(ws + L.order_off) : nullptr;
  p->recs = ws + L.table_bytes;
  p->bbuf = L.m_off > L.b_off ? (float*)(ws + L.b_off) : nullptr;
  p->mbuf = L.total_bytes > L.m_off ? (uint16_t*)(ws + L.m_off) : nullptr;
  p->seg_L = L.seg_L;
  p->seg_S = L.seg_S;
  p->max_segs = L.max_segs;
  p->seg_path = L.seg_path;
  p->scale = a->scale;
  p->B = a->B; p->T = a->T; p->HQK = a->HQK; p->HV = a->HV; p->K = a->K; p->V = a->V; p->N = a->N;
  p->NT = (int)(((int64_t)a->T + kda::BT - 1) / kda::BT);
  p->max_chunks = L.max_chunks;
  return KDA_OK;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return KDA_OK;
  strncpy(g_hip_msg, hipGetErrorString(e), sizeof(g_hip_msg) - 1);
  g_hip_msg[sizeof(g_hip_msg) - 1] = 0;
  return KDA_ERR_HIP;
}

// Workspace layout of the backward scan: [varlen: chunk table (N + 2 int32), segment table
// (N + 1, segmented scan), longest-first order (N, when each sequence is one scan unit and
// N <= ORDER_MAX_N) | pad to 256 | b | M] (b and M only when a sequence has several segments).
struct BwdLayout {
  bool seg_path;
  int seg_L, seg_S;
  int64_t max_segs;
  int64_t segtab_off, order_off;   // byte offsets, or -1
  int64_t b_off, m_off, total;
};

// Shape checks of the backward scan and its plan (the forward's rule, kda_plan.hpp).
int check_bwd_shapes(const kda_bwd_dhu_args* a, BwdLayout* L) {
  if (!a) return KDA_ERR_INVALID_ARG;
  if (a->K != 64 && a->K != 128) return KDA_ERR_UNSUPPORTED;
  if (a->V <= 0 || a->V % kda::BV != 0) return KDA_ERR_UNSUPPORTED;
  if (a->B < 1 || a->T < 0 || a->HV < 1 || a->N < 1) return KDA_ERR_INVALID_ARG;
  if (a->seg_chunks < 0) return KDA_ERR_INVALID_ARG;
  if (a->cu_seqlens) {
    if (a->B != 1) return KDA_ERR_INVALID_ARG;
  } else if (a->N != a->B) {
    return KDA_ERR_INVALID_ARG;
  }
  if ((int64_t)a->B * a->T > ((int64_t)1 << 40)) return KDA_ERR_INVALID_ARG;
  const int64_t nt = ((int64_t)a->T + kda::BT - 1) / kda::BT;
  const int64_t max_chunks = a->cu_seqlens ? nt + a->N : (int64_t)a->B * nt;
  if (max_chunks * a->HV >= ((int64_t)1 << 31) - 8) return KDA_ERR_INVALID_ARG;
  if ((int64_t)a->N * a->HV * (a->V / kda::BV) >= ((int64_t)1 << 31) - 8) return KDA_ERR_INVALID_ARG;
  if (a->N >= (1 << 30)) return KDA_ERR_INVALID_ARG;
  const kda::ScanPlan plan = kda::choose_scan(nt, a->cu_seqlens != nullptr, a->N, a->HV, a->V,
                                              a->seg_chunks > 0 ? 0 : kda::device_cus(), a->seg_chunks);
  L->seg_path = plan.seg_path;
  const int64_t seg_L = std::min<int64_t>(plan.seg_L, std::max<int64_t>(nt, 1));
  int64_t seg_S = 1, max_segs = 0;
  bool multi = false;
  if (plan.seg_path) {
    if (a->cu_seqlens) {
      max_segs = (nt + a->N) / seg_L + a->N;
      multi = seg_L < nt;
    } else {
      seg_S = std::max<int64_t>(1, (nt + seg_L - 1) / seg_L);
      max_segs = (int64_t)a->B * seg_S;
      multi = seg_S > 1;
    }
    if (max_segs * a->HV * ((a->V + 63) / 64 + a->K / 64) >= ((int64_t)1 << 31) - 8) return KDA_ERR_INVALID_ARG;
  }
  L->seg_L = (int)seg_L;
  L->seg_S = (int)seg_S;
  L->max_segs = max_segs;
  L->segtab_off = L->order_off = -1;
  int64_t head = 0;
  if (a->cu_seqlens) {
    head = ((int64_t)a->N + 2) * 4;
    if (plan.seg_path) {
      L->segtab_off = head;
      head += ((int64_t)a->N + 1) * 4;
    }
    if (!multi && a->N <= kda::ORDER_MAX_N) {
      L->order_off = head;
      head += (int64_t)a->N * 4;
    }
  }
  const int64_t bbytes = multi ? max_segs * a->HV * a->K * a->V * 4 : 0;
  const int64_t mbytes = multi ? max_segs * a->HV * a->K * a->K * 2 : 0;
  L->b_off = (head + 255) / 256 * 256;
  L->m_off = L->b_off + bbytes;
  L->total = (head == 0 && bbytes == 0) ? 0 : L->m_off + mbytes;
  return KDA_OK;
}

// Device address of `scratch` on the current device, looked up once per device (the
// first call on a device makes it; concurrent first calls look up the same address).
constexpr int MAX_DEVICES = 64;
std::atomic<uint8_t*> g_scratch[MAX_DEVICES];

int scratch_on_current_device(uint8_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= MAX_DEVICES) return KDA_ERR_UNSUPPORTED;
  uint8_t* ptr = g_scratch[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    void* sym = nullptr;
    e = hipGetSymbolAddress(&sym, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e);
    if (sym == nullptr || !aligned(sym, 256)) return KDA_ERR_WORKSPACE;
    ptr = static_cast<uint8_t*>(sym);
    g_scratch[dev].store(ptr, std::memory_order_release);
  }
  *out = ptr;
  return KDA_OK;
}

int run_intra(const kda::Params& p, hipStream_t s) {
  if (p.max_chunks * p.HV == 0) return KDA_OK;
  int st = hip_status(p.cu ? kda::launch_chunk_table(p.cu, p.N, p.T, p.max_chunks, p.table, p.counter, p.seg_L,
                                                     p.max_segs, p.segtab, p.cinfo, p.order, s)
                           : kda::launch_prep(p, s));
  if (st != KDA_OK) return st;
  return hip_status(kda::launch_intra(p, s));
}

}  // namespace

extern "C" {

int kda_fwd_workspace_bytes(const kda_fwd_args* a, size_t* bytes) {
  if (!bytes) return KDA_ERR_INVALID_ARG;
  kda::WsLayout L;
  int st = check_shapes(a, &L);
  if (st != KDA_OK) return st;
  *bytes = (size_t)L.total_bytes;
  return KDA_OK;
}

int kda_fwd_scan_plan(const kda_fwd_args* a, int32_t* seg_chunks) {
  if (!seg_chunks) return KDA_ERR_INVALID_ARG;
  kda::WsLayout L;
  int st = check_shapes(a, &L);
  if (st != KDA_OK) return st;
  *seg_chunks = L.seg_path ? L.seg_L : 0;
  return KDA_OK;
}

int kda_fwd_intra(const kda_fwd_args* a) {
  kda::Params p;
  int st = check_call(a, NEED_INTRA, &p);
  if (st != KDA_OK) return st;
  return run_intra(p, (hipStream_t)a->stream);
}

int kda_fwd_inter(const kda_fwd_args* a) {
  kda::Params p;
  int st = check_call(a, NEED_INTER, &p);
  if (st != KDA_OK) return st;
  return hip_status(p.seg_path ? kda::launch_scan(p, (hipStream_t)a->stream) : kda::launch_inter(p, (hipStream_t)a->stream));
}

int kda_fwd(const kda_fwd_args* a) {
  kda::Params p;
  int st = check_call(a, NEED_INTRA | NEED_INTER, &p);
  if (st != KDA_OK) return st;
  st = run_intra(p, (hipStream_t)a->stream);
  if (st != KDA_OK) return st;
  return hip_status(p.seg_path ? kda::launch_scan(p, (hipStream_t)a->stream) : kda::launch_inter(p, (hipStream_t)a->stream));
}

int kda_fwd_no_alloc(const kda_fwd_args* a) {
  if (!a) return KDA_ERR_INVALID_ARG;
  kda::WsLayout L;
  int st = check_shapes(a, &L);
  if (st != KDA_OK) return st;
  if ((uint64_t)L.total_bytes > (uint64_t)KDA_NO_ALLOC_MAX_BYTES) return KDA_ERR_TOO_LARGE;
  // every argument is checked before the scratch is looked up (a HIP call)
  st = check_args(a, NEED_INTRA | NEED_INTER, &L);
  if (st != KDA_OK) return st;
  uint8_t* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st != KDA_OK) return st;
  kda_fwd_args b = *a;
  b.workspace = ws;
  b.workspace_bytes = KDA_NO_ALLOC_MAX_BYTES;
  return kda_fwd(&b);
}

int kda_debug_unpack(const kda_fwd_args* a, void* qg, void* w, void* kg, void* aqk, void* tmb,
                     float* alpha) {
  kda::Params p;
  int st = check_call(a, 0, &p);
  if (st != KDA_OK) return st;
  if (p.c16) return KDA_ERR_UNSUPPORTED;   // the unpacked layout is that of chunk 64
  const void* outs[] = {qg, w, kg, aqk, tmb, alpha};
  for (const void* ptr : outs)
    if (!aligned(ptr, 16)) return KDA_ERR_INVALID_ARG;
  return hip_status(kda::launch_unpack(p, (uint16_t*)qg, (uint16_t*)w, (uint16_t*)kg, (uint16_t*)aqk,
                                       (uint16_t*)tmb, alpha, (hipStream_t)a->stream));
}

int kda_bwd_dhu_workspace_bytes(const kda_bwd_dhu_args* a, size_t* bytes) {
  if (!bytes) return KDA_ERR_INVALID_ARG;
  BwdLayout L;
  int st = check_bwd_shapes(a, &L);
  if (st != KDA_OK) return st;
  *bytes = (size_t)L.total;
  return KDA_OK;
}

int kda_bwd_dhu(const kda_bwd_dhu_args* a) {
  BwdLayout L;
  int st = check_bwd_shapes(a, &L);
  if (st != KDA_OK) return st;
  const int64_t ws = L.total;
  if ((int64_t)a->B * a->T > 0 && (!a->qg || !a->kg || !a->w || !a->g2 || !a->dout || !a->dv2))
    return KDA_ERR_INVALID_ARG;
  const void* a16[] = {a->qg, a->kg, a->w, a->g2, a->dht, a->dh0, a->dhc};
  for (const void* ptr : a16)
    if (!aligned(ptr, 16)) return KDA_ERR_INVALID_ARG;
  const void* a8[] = {a->dout, a->dv, a->dv2, a->cu_seqlens};
  for (const void* ptr : a8)
    if (!aligned(ptr, 8)) return KDA_ERR_INVALID_ARG;
  if (a->flags & ~(uint32_t)(KDA_FLAG_STATE_BF16 | KDA_FLAG_CKPT_BF16)) return KDA_ERR_INVALID_ARG;
  if (ws > 0 && (!a->workspace || !aligned(a->workspace, 256) || a->workspace_bytes < (size_t)ws))
    return KDA_ERR_WORKSPACE;
  if (!(a->scale == a->scale)) return KDA_ERR_INVALID_ARG;
  kda::BwdParams p;
  p.qg = (const uint16_t*)a->qg;
  p.kg = (const uint16_t*)a->kg;
  p.w = (const uint16_t*)a->w;
  p.g2 = a->g2;
  p.dout = (const uint16_t*)a->dout;
  p.dv = (const uint16_t*)a->dv;
  p.dht = a->dht;
  p.cu = a->cu_seqlens;
  p.dv2 = (uint16_t*)a->dv2;
  p.dh0 = a->dh0;
  p.dhc = a->dhc;
  uint8_t* ws8 = (uint8_t*)a->workspace;
  p.table = a->cu_seqlens ? (int32_t*)ws8 : nullptr;
  p.segtab = L.segtab_off >= 0 ? (int32_t*)(ws8 + L.segtab_off) : nullptr;
  p.order = L.order_off >= 0 ? (int32_t*)(ws8 + L.order_off) : nullptr;
  p.bbuf = L.m_off > L.b_off ? (float*)(ws8 + L.b_off) : nullptr;
  p.mbuf = L.total > L.m_off ? (uint16_t*)(ws8 + L.m_off) : nullptr;
  p.seg_path = L.seg_path;
  p.seg_L = L.seg_L;
  p.seg_S = L.seg_S;
  p.max_segs = L.max_segs;
  p.scale = a->scale;
  p.flags = a->flags;
  p.B = a->B; p.T = a->T; p.HV = a->HV; p.K = a->K; p.V = a->V; p.N = a->N;
  p.NT = (int)(((int64_t)a->T + kda::BT - 1) / kda::BT);
  hipStream_t s = (hipStream_t)a->stream;
  if (a->cu_seqlens) {
    const int64_t cap = p.NT + (int64_t)p.N;   // upper bound on the chunk count
    st = hip_status(kda::launch_chunk_table(p.cu, p.N, p.T, cap, p.table, nullptr, L.seg_path ? L.seg_L : 1,
                                            L.max_segs, p.segtab, nullptr, p.order, s));
    if (st != KDA_OK) return st;
  }
  return hip_status(p.seg_path ? kda::launch_bwd_scan(p, s) : kda::launch_bwd_dhu(p, s));
}

const char* kda_strerror(int status) {
  switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, bad size or head counts)";
    case KDA_ERR_UNSUPPORTED: return "unsupported shape (K must be 64 or 128, V a positive multiple of 16)";
    case KDA_ERR_WORKSPACE: return "workspace missing, not 256-byte aligned, or smaller than kda_fwd_workspace_bytes";
    case KDA_ERR_HIP: return g_hip_msg;
    case KDA_ERR_TOO_LARGE:
      return "the shapes need more scratch than kda_fwd_no_alloc's static buffer (KDA_NO_ALLOC_MAX_BYTES) holds; "
             "call kda_fwd with a workspace";
    default: return "unknown status";
  }
}

}  // extern "C"
