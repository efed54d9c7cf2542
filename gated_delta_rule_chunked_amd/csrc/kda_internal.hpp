// kda_internal.hpp -- kernel parameters and host-side launch entry points shared
// by the C ABI (kda_api.cpp) and the kernel files.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// kda_fwd_args.flags / kda_bwd_dhu_args.flags bits (same values as KDA_FLAG_* in include/kda.h)
constexpr uint32_t FLAG_BETA_LOGITS = 1u;
constexpr uint32_t FLAG_STATE_BF16 = 2u;
constexpr uint32_t FLAG_CKPT_BF16 = 4u;

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* g;
  const uint16_t* beta;
  const void* h0;       // fp32, or bf16 with KDA_FLAG_STATE_BF16
  const int64_t* cu;     // varlen cu_seqlens or nullptr
  uint16_t* o;
  void* ht;             // state dtype
  int32_t* table;        // varlen: chunk_base[N+1], then error flag at [N+1]
  int32_t* counter;      // work counter of the intra stage (zeroed by the prep kernel)
  int2* cinfo;           // varlen: per chunk {first row, valid rows}, else nullptr
  void* hc;              // per-chunk states (state dtype) or nullptr
  uint8_t* recs;         // workspace records
  float scale;
  uint32_t flags;        // KDA_FLAG_* bits
  bool c16;              // chunk length 16 (four 16-row chunks per 64-row record), else 64
  int B, T, HQK, HV, K, V, N;
  int NT;                // fixed length: chunks per sequence
  int64_t max_chunks;    // workspace capacity in chunks (per value head)
  // Segmented scan: each sequence is cut into segments of seg_L chunks that are
  // scanned in parallel (kda_scan.hip).
  bool seg_path;         // the segmented scan runs (kda_scan.hip), else the serial one (kda_inter.hip)
  int seg_L;             // chunks per segment
  int seg_S;             // fixed length: segments per sequence
  int64_t max_segs;      // capacity of the segment buffers (segments over all sequences)
  int32_t* segtab;       // varlen: seg_base[N+1] in the workspace header, else nullptr
  int32_t* order;        // varlen, one segment per sequence: sequences longest first, else nullptr
  float* bbuf;           // K x V fp32 segment end states per (segment, HV), in the column
                         // waves' C-layout order (kda_scan.hip), or nullptr (one segment)
  uint16_t* mbuf;        // K x K bf16 segment transitions per (segment, HV), as P-order A
                         // fragments (kda_scan.hip), or nullptr
};

// Reverse state scan of the backward (kda_bwd_dhu).
struct BwdParams {
  const uint16_t* qg;    // bf16 [B, T, HV, K]
  const uint16_t* kg;
  const uint16_t* w;
  const float* g2;       // fp32 [B, T, HV, K], chunk-local cumsum of g in log2 units
  const uint16_t* dout;  // bf16 [B, T, HV, V]
  const uint16_t* dv;    // bf16 [B, T, HV, V] or nullptr (zero)
  const void* dht;       // state dtype, or nullptr
  const int64_t* cu;
  uint16_t* dv2;         // bf16 [B, T, HV, V]
  void* dh0;             // state dtype, or nullptr
  void* dhc;             // checkpoint dtype, or nullptr
  int32_t* table;        // varlen chunk table (workspace) or nullptr
  int32_t* order;        // varlen, one scan unit per sequence: sequences longest first, or nullptr
  float scale;
  uint32_t flags;        // FLAG_STATE_BF16, FLAG_CKPT_BF16
  int B, T, HV, K, V, N;
  int NT;                // fixed length: chunks per sequence
  // Segmented 64-column scan (kda_bwd_scan.hip), the same plan as the forward's
  bool seg_path;         // the segmented scan runs, else the 16-column serial one (kda_bwd.hip)
  int seg_L;             // chunks per segment
  int seg_S;             // fixed length: segments per sequence
  int64_t max_segs;      // capacity of the segment buffers
  int32_t* segtab;       // varlen: seg_base[N+1] (workspace), else nullptr
  float* bbuf;           // K x V fp32 per (segment, HV): the dh a segment hands to the next older one
  uint16_t* mbuf;        // K x K bf16 per (segment, HV): the segment's transition, as P-order A fragments
};

// Host launchers (return the hipError_t of the launch).
// varlen chunk table (chunk_base[N+1], error flag at [N+1]); also zeroes *counter when
// non-null, writes seg_base[N+1] (segments of seg_L chunks, at least one per
// sequence) when segtab is non-null and per-chunk {first row, valid rows} when
// cinfo is non-null, and the sequences ordered by chunk count, longest first, when
// order is non-null (N <= ORDER_MAX_N)
hipError_t launch_chunk_table(const int64_t* cu, int N, int T, int64_t max_chunks, int32_t* table,
                              int32_t* counter, int seg_L, int64_t max_segs, int32_t* segtab, int2* cinfo,
                              int32_t* order, hipStream_t s);
constexpr int ORDER_MAX_N = 2048;   // longest-first order: sorted on one workgroup up to this many sequences
int device_cus();                                               // compute units of the current device
hipError_t launch_prep(const Params& p, hipStream_t s);          // fixed length: zeroes the counter
hipError_t launch_intra(const Params& p, hipStream_t s);
hipError_t launch_inter(const Params& p, hipStream_t s);
hipError_t launch_scan(const Params& p, hipStream_t s);          // segmented scan (both passes)
hipError_t launch_bwd_dhu(const BwdParams& p, hipStream_t s);
hipError_t launch_bwd_scan(const BwdParams& p, hipStream_t s);   // segmented scan (both passes)
hipError_t launch_unpack(const Params& p, uint16_t* qg, uint16_t* w, uint16_t* kg,
                         uint16_t* aqk, uint16_t* tmb, float* alpha, hipStream_t s);

}  // namespace kda
