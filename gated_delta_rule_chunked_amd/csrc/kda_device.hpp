// kda_device.hpp -- device helpers and the workspace record layout shared by the
// intra-chunk and inter-chunk kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

constexpr int BT = 64;        // chunk length (tokens)
constexpr int BV = 16;        // value columns per inter-chunk workgroup
constexpr int NTHREADS = 256; // 4 waves per workgroup, both kernels
constexpr float LOG2E = 1.4426950408889634f;

typedef short bf16x8 __attribute__((ext_vector_type(8)));
typedef short bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2n __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ MFMA
// v_mfma_f32_16x16x32_bf16, lane l = 16*g + r (g = l/16, r = l%16):
//   A (16 x 32): lane holds A[r][8g .. 8g+7]
//   B (32 x 16): lane holds B[8g .. 8g+7][r]
//   C (16 x 16): lane holds C[4g .. 4g+3][r]
__device__ __forceinline__ f32x4 mfma16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// v_mfma_f32_16x16x16_bf16: A lane holds A[r][4g .. 4g+3], B lane holds B[4g .. 4g+3][r]
// (either half of a P-order 32-step fragment, or a packed C-layout tile as B).
__device__ __forceinline__ f32x4 mfma16x16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// v_mfma_f32_16x16x4_f32 (fp32 operands): A lane holds A[r][g], B lane holds
// B[g][r], C as above.
__device__ __forceinline__ f32x4 mfma16x4f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ bf16
// Bits of a float, taken by value.  With this compiler, __builtin_bit_cast applied
// directly to an ext_vector element (v[i]) reads element 0 whatever i is, so
// vector elements go through this copy.
__device__ __forceinline__ uint32_t f2u(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float bf2f(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}
__device__ __forceinline__ float bflo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bfhi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }
// Two floats -> packed bf16 pair (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2n));
}
__device__ __forceinline__ uint16_t f2bf(float x) { return (uint16_t)(pack2(x, 0.f) & 0xffffu); }

// 8 bf16 (one uint4) <-> 8 floats
__device__ __forceinline__ void unpack8(const uint4& u, float* f) {
  f[0] = bflo(u.x); f[1] = bfhi(u.x); f[2] = bflo(u.y); f[3] = bfhi(u.y);
  f[4] = bflo(u.z); f[5] = bfhi(u.z); f[6] = bflo(u.w); f[7] = bfhi(u.w);
}
__device__ __forceinline__ uint4 pack8(const float* f) {
  return make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7]));
}
__device__ __forceinline__ bf16x8 as_frag(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }

// 16-byte store with the non-temporal hint (global_store ... nt).  The intra stage
// writes its workspace records this way: each record is written once and read
// back only by the scan kernel, and the scan runs measurably faster on records
// stored with the hint than on records left in the caches by ordinary stores.
typedef uint32_t u32x4n __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_stream(void* dst, const uint4& v) {
  __builtin_nontemporal_store(u32x4n{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4n*>(dst));
}

// ------------------------------------------------------------ DPP scans
// Inclusive prefix sum over the 16 lanes of each DPP row (lanes 16g .. 16g+15),
// in lane order.  row_shr:n moves lane i-n to lane i inside a row; lanes with
// no source receive 0 (bound_ctrl).
template <int N>
__device__ __forceinline__ float row_shr(float x) {
  int v = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + N, 0xf, 0xf, true);
  return __builtin_bit_cast(float, v);
}
__device__ __forceinline__ float row_inclusive_scan(float x) {
  x += row_shr<1>(x);
  x += row_shr<2>(x);
  x += row_shr<4>(x);
  x += row_shr<8>(x);
  return x;
}

// ----------------------------------------------------- block -> XCD remap
// Workgroups are dispatched round-robin over the 8 XCDs (block b runs on XCD
// b % 8).  Remapping makes consecutive logical ids share an XCD and its L2, so
// the value tiles of one head (inter kernel) and the two value heads of one q/k
// head (intra kernel) meet in the same L2.  Correctness never depends on it.
// `grid` must be a multiple of 8.
__device__ __forceinline__ int xcd_remap(int b, int grid) {
  return (b & 7) * (grid >> 3) + (b >> 3);
}

// -------------------------------------------------------------- P-order
// Every MFMA fragment that contracts over a 32-wide step uses "P-order": lane
// group g (lanes 16g .. 16g+15) supplies the contraction indices
//   {4g, 4g+1, 4g+2, 4g+3, 16+4g, 16+4g+1, 16+4g+2, 16+4g+3}   (step-relative)
// in that register order.  The 16x16 C layout gives lane group g rows 4g .. 4g+3
// of each 16-row tile, so a result tile pair (rows 0-15 and 16-31 of the step)
// becomes an A or B fragment without moving data between lanes.
__device__ __forceinline__ constexpr int pidx(int g, int e) { return 4 * g + (e & 3) + ((e >> 2) << 4); }

// 8 bf16 of a P-order fragment from a bf16 row whose contraction index is
// contiguous: two 8-byte reads at base + 4g and base + 16 + 4g.
__device__ __forceinline__ bf16x8 pfrag(const uint16_t* row, int base, int g) {
  const uint2 lo = *reinterpret_cast<const uint2*>(row + base + 4 * g);
  const uint2 hi = *reinterpret_cast<const uint2*>(row + base + 16 + 4 * g);
  return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}
// Two C-layout tiles (4 floats each) -> one packed P-order fragment.
__device__ __forceinline__ uint4 pack_pair(const f32x4& lo, const f32x4& hi) {
  return make_uint4(pack2(lo[0], lo[1]), pack2(lo[2], lo[3]), pack2(hi[0], hi[1]), pack2(hi[2], hi[3]));
}

// ------------------------------------------------------- scan helpers
// Raw barrier: the wave's own LDS writes complete, then s_barrier, with a compiler
// memory clobber.  __syncthreads would also wait for every outstanding global load
// of the wave, which would serialize the register rings.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// State tensors are fp32, or bf16 when `bf16` is set.
__device__ __forceinline__ float load_state(bool bf16, const void* base, int64_t idx) {
  return bf16 ? bf2f(static_cast<const uint16_t*>(base)[idx]) : static_cast<const float*>(base)[idx];
}
__device__ __forceinline__ void store_state(bool bf16, void* base, int64_t idx, float x) {
  if (bf16) static_cast<uint16_t*>(base)[idx] = f2bf(x);
  else static_cast<float*>(base)[idx] = x;
}

__device__ __forceinline__ uint2 pack4(const f32x4& a) {
  return make_uint2(pack2(a[0], a[1]), pack2(a[2], a[3]));
}
__device__ __forceinline__ bf16x8 cat(const uint2& lo, const uint2& hi) {
  return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}
__device__ __forceinline__ bf16x4 as_half(const uint2& u) { return __builtin_bit_cast(bf16x4, u); }
__device__ __forceinline__ uint2 lds8(const uint8_t* p) { return *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ uint4 lds16(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }

// One sequence of a scan workgroup: batch row, first row, length, and the index
// of its first chunk in the chunk numbering shared by the per-chunk outputs.
struct SeqLoc {
  int b;
  int64_t bos;
  int len;
  int64_t cbase;  // chunk index of the sequence's first chunk
};

// One segment of one sequence (segmented scans: chunks c0 .. c0 + ncs - 1 of it).
struct SegLoc {
  int n, s, nseg;       // sequence, segment within it, its segment count
  int64_t sigma0;       // index of the sequence's first segment
  int b;                // batch row
  int64_t bos;          // first row of the sequence within the batch row
  int len;              // tokens of the sequence
  int64_t cbase;        // chunk index of the sequence's first chunk
  int c0, ncs;          // first chunk of the segment (within the sequence), chunks in it
};

// Segment sigma -> location.  Returns false when sigma is past the last segment.
// Works on the forward and the backward parameter blocks (same field names).
template <class P>
__device__ __forceinline__ bool locate_segment(const P& p, int64_t sigma, SegLoc& sl) {
  if (p.cu == nullptr) {
    const int64_t n = sigma / p.seg_S;
    if (n >= p.B) return false;
    sl.n = (int)n;
    sl.s = (int)(sigma - n * p.seg_S);
    sl.nseg = p.seg_S;
    sl.sigma0 = n * p.seg_S;
    sl.b = (int)n;
    sl.bos = 0;
    sl.len = p.T;
    sl.cbase = n * p.NT;
  } else {
    if (sigma >= p.segtab[p.N]) return false;
    int lo = 0, hi = p.N;                      // segtab[lo] <= sigma < segtab[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.segtab[mid] <= sigma) lo = mid;
      else hi = mid;
    }
    sl.n = lo;
    sl.sigma0 = p.segtab[lo];
    sl.s = (int)(sigma - sl.sigma0);
    sl.nseg = p.segtab[lo + 1] - p.segtab[lo];
    sl.b = 0;
    sl.bos = p.cu[lo];
    sl.len = (int)(p.cu[lo + 1] - p.cu[lo]);
    sl.cbase = p.table[lo];
  }
  const int nc = (sl.len + BT - 1) / BT;
  sl.c0 = sl.s * p.seg_L;
  sl.ncs = max(0, min(p.seg_L, nc - sl.c0));
  return true;
}

// ds_read_b64_tr_b16, the gfx950 LDS transpose read (8 bytes per lane).  Within
// each block of 16 lanes, lane 4a + e receives as its element j (a, e, j = 0..3)
// element e of the 8 bytes addressed by lane 4j + a of the block (lane layout
// measured on gfx950).  On a row-major 16-bit tile, with lane (b = l/16, j, a) of
// the wave addressing row row0 + 4b + j, columns col0 + 4a .. +3, lane (g, r)
// receives rows row0 + 4g .. +3 of column col0 + r: a 16x16 C-layout tile, or the
// low (high) half of a P-order fragment that contracts over the tile's rows.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_tr8(const uint8_t* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(uint2, v);
}

// ---------------------------------------------------- workspace records
// One record per (chunk, value head), written by the intra kernel in the exact
// register-fragment order the inter kernel consumes (64 lanes x 16 B per
// fragment, so every operand fragment is one contiguous 1 KiB).  All fragments
// are in P-order along their contraction index.
//
//   WN  : A operand of  v' = u + (-w) h   [64 x K] bf16 (negated w)
//   KGT : A operand of  DH = kg^T v'  [K x 64] bf16
//   TMB : A operand of  u = (Tm diag beta) v   [64 x 64] bf16 lower triangle
//   ALPHA: exp2(G) per key dimension, fp32 [K]
//   QG  : A operand of  O = qg h     [64 x K] bf16, scale folded in
//   AQK : A operand of  O += Aqk v'   [64 x 64] bf16 lower triangle
// The state-update operands (WN, KGT, TMB, ALPHA) come first and are contiguous
// (STATE_BYTES), so the scan stages them into LDS as one block copy.
//
// [64 x K] fragments (QG, WN): frag (mb, s), mb = row block 0..3, s = 32-column
//   step 0..K/32-1; lane l holds row 16mb + l%16 and columns 32s + pidx(l/16, e).
//   byte offset ((mb * K/32 + s) * 64 + l) * 16.
// KGT fragments: frag (md, s), md = 16-row block of the key dimension 0..K/16-1,
//   s = 0,1 (token halves); lane l holds d = 16md + l%16, tokens 32s + pidx(l/16, e).
//   byte offset ((md * 2 + s) * 64 + l) * 16.
// AQK / TMB: lower-triangular 64 x 64, the two all-zero fragments (rows 0..31,
//   columns 32..63) are not stored: frag index (mb, s) -> {0,1,2,3,4,5} for
//   (0,0),(1,0),(2,0),(2,1),(3,0),(3,1); lane layout as QG.
// A P-order 32-step fragment is also two 16x16x16 fragments: its low 8 bytes
// cover indices 4g..4g+3 of the first 16, its high 8 bytes those of the second.
template <int K>
struct Rec {
  static constexpr int S = K / 32;                 // 32-wide K steps
  static constexpr int WN = 0;
  static constexpr int KGT = WN + BT * K * 2;
  static constexpr int TMB = KGT + BT * K * 2;
  static constexpr int ALPHA = TMB + 6 * 1024;
  static constexpr int STATE_BYTES = ALPHA + K * 4;   // 39424 (K=128), 22784 (K=64)
  static constexpr int QG = STATE_BYTES;
  static constexpr int AQK = QG + BT * K * 2;
  static constexpr int BYTES = AQK + 6 * 1024;     // 61952 (K=128), 37120 (K=64)
  static_assert(BYTES % 256 == 0 && STATE_BYTES % 256 == 0, "records stay 256-byte aligned");
};
// Chunk 16 (FlashKDA's chunk length) uses the same records: one per 64 rows, holding
// four 16-row chunks whose Aqk and Tm diag(beta) are block diagonal, so fragments
// (2,0) and (3,0) of AQK and TMB are zero and never read.  The decay rows exp2(G) of
// sub-chunks 1..3 live in those two TMB fragments (part of the state block, so the
// state pass stages them); sub-chunk 0's is the ALPHA row.
template <int K>
__device__ __host__ __forceinline__ constexpr int alpha16_off(int I) {
  return I == 0 ? Rec<K>::ALPHA
                : Rec<K>::TMB + (((I - 1) * K) / 256 == 0 ? 2 : 4) * 1024 + (((I - 1) * K) % 256) * 4;
}
static_assert(alpha16_off<128>(3) + 128 * 4 <= Rec<128>::TMB + 5 * 1024 && alpha16_off<64>(3) + 64 * 4 <= Rec<64>::TMB + 3 * 1024,
              "chunk-16 decay rows stay inside the zero TMB fragments");

// Records are stored chunk-major: the HV records of one chunk are contiguous.
// The scans run consecutive heads side by side at the same chunk position, so
// the records in flight at one time sit next to each other instead of being
// max_chunks records apart, which spreads the streams over the memory
// channels more evenly than head-major storage did.
__device__ __host__ __forceinline__ int64_t rec_index(int hv, int64_t chunk, int64_t nheads) {
  return chunk * nheads + hv;
}
__device__ __host__ __forceinline__ constexpr int tri_frag(int mb, int s) {
  return mb < 2 ? mb : 2 * mb - 2 + s;   // (0,0)0 (1,0)1 (2,0)2 (2,1)3 (3,0)4 (3,1)5
}
__device__ __host__ __forceinline__ constexpr int tri_steps(int mb) { return mb < 2 ? 1 : 2; }

// Layout of the workspace: [header | records | 1 KiB pad | B | M].  Header: int32
// work counter of the intra stage at byte 0; for varlen, the chunk table (int32
// chunk_base[N+1]) and an int32 error flag from byte 16, then (segmented scan) the
// segment table (int32 seg_base[N+1]) and, 8-byte aligned, int32 {first row, valid
// rows} per chunk; padded to a multiple of 256 bytes.  The pad keeps the scan's
// whole-KiB record copies inside the workspace.  B (fp32, K x V per segment and HV) and
// M (bf16, K x K per segment and HV) hold the segmented scan's per-segment end states and
// transitions; they are empty when no sequence has more than one segment.
struct WsLayout {
  int64_t table_bytes;  // header: counter, varlen chunk table, segment table and chunk info
  int64_t cinfo_off;    // varlen: byte offset of the per-chunk {first row, valid rows}
  int64_t rec_bytes;
  int64_t max_chunks;   // capacity in chunks per value head
  int64_t b_off, m_off; // segment end states / transitions (0 bytes when every sequence is one segment)
  int64_t total_bytes;
  bool seg_path;        // the segmented scan is used
  int seg_L, seg_S;     // chunks per segment; fixed length: segments per sequence
  int64_t max_segs;
  int64_t order_off;    // varlen, one segment per sequence: byte offset of the longest-first
                        // sequence order (int32 [N]), or 0 when the scan keeps the given order
};

}  // namespace kda
