// Paged / segmented attention kernels for gfx950 (CDNA4, wave64, MFMA).
//
// Rows of a work item are the G query heads of one kv head times the query
// block (row r -> token r / G, head kvh*G + r % G), packed into 16-row MFMA
// tiles.  Keys are consumed in tiles of 16 slots of one page (paged modes; the
// dense fp8-query block pairs two such tiles), of one segment (segment
// partials), or of a query's live keys numbered across its segments (fused
// segments: a tile may span segments).
//
// Per 16-key tile and 16-row tile:
//   S^T = K Q^T      D/32 x v_mfma_f32_16x16x32_{bf16,f16}, or _fp8_fp8 on the
//                    stored bytes of K and q for an fp8 query; K is the A
//                    operand (lane l: key l%16, 16 contiguous bytes of its row).
//   online softmax   fp32 registers, log2 domain, v_exp_f32.
//   O^T += V^T P^T   D/16 x v_mfma_f32_16x16x16_{bf16,f16}; P^T is the S^T
//                    accumulator re-packed to 16 bits in place (same lane
//                    layout).  V^T: in attn_kernel from 4 keys x VPL head-dim
//                    values per lane with 16-bit permutes (A-row m of MFMA j is
//                    head-dim VPL*m + j); in attn_shared_kernel from transposing
//                    LDS reads (A-row m of MFMA j is head-dim 16*j + m).
// fp8 (e4m3fn) K/V are decoded exactly to the 16-bit P.V type with the gfx950
// pk conversions (K too, unless the query is fp8); k_scale folds into the logit
// scale and v_scale into the epilogue (vllm.v1.attention.backends.flashinfer_ts,
// forward: bmm1_scale / bmm2_scale).  Both kernels also come in a causal form:
// bottom-right causal rows with an exact per-token window.
//
// Three kernels:
//   attn_kernel         waves of a workgroup split the KEYS (round-robin
//                       tiles, K/V loaded straight into registers one tile
//                       ahead) and merge their softmax states through LDS.
//                       Used for <= 16 rows (decode) and the segment modes.
//   dash_shared_kernel  fused segments: one workgroup per (query, pair of kv
//                       heads), one wave per head, the pair's token rows
//                       staged through a two-stage LDS ring.
//   attn_shared_kernel  waves split the ROWS (one 16-row tile each) and all
//                       consume the same K/V tiles, which stream through an
//                       NBUF-stage LDS ring filled by direct-to-LDS loads
//                       (global_load_lds_dwordx4): one HBM read per tile, no
//                       VGPR staging, NBUF-1 tiles in flight.  Used for query
//                       blocks with more than 16 rows.

#include <type_traits>

#include "pa_device.h"
#include "pa_kernels.h"
#include "pa_plan.h"

namespace pa {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRescaleSlack = 8.0f;  // log2 units: softmax terms stay <= 256 before a rescale
// attend_tile's optional hooks: `mid` runs right after the S^T MFMAs are
// issued, `vload` fills the V^T operands right before the P.V MFMAs
struct NoHook {
  __device__ void operator()() const {}
};

template <int D, int KV>
struct Geo {
  static constexpr int KB = (KV == K_FP8) ? 1 : 2;  // bytes per stored K/V element
  static constexpr int NKC = D / 32;                // QK MFMAs per row tile
  static constexpr int VPL = D / 16;                // PV MFMAs per row tile
  static constexpr int KLD = D * KB / 64;           // 16-byte K pieces per lane per tile
  static constexpr int VB = VPL * KB;               // V bytes per lane per key
  static constexpr int VDW = VB / 4;                // ... in dwords
  static constexpr int RB = 2 * D * KB;             // bytes of one key's K and V in a staged tile
  static constexpr int CPK = RB / 16;               // 16-byte chunks per staged key
  static constexpr int SWZ = CPK / 2 - 1;           // chunk swizzle mask within the K or V half
  // XOR applied to the chunk numbers of key t in a staged tile: t for K
  // chunks; 2t for the V chunks of a 16-bit cache, so that the transposing V
  // reads of one half-wave (keys t..t+7, two adjacent chunks each) land on 16
  // distinct chunk positions instead of 8.
  __device__ static int swz(int t, int c) {
    if constexpr (KV == K_FP8 && CPK == 16) {
      // 256-byte rows: a mask that also swaps the K and V halves of keys
      // 4..7 and 12..15 (bit 3), so the K reads and the 8-bit transposing V
      // reads each cover every bank instead of the half their chunks sit in
      return ((2 * t) & 6) | (((t >> 2) ^ (t >> 3)) & 1) | (((t >> 2) & 1) << 3);
    }
    if (KV != K_FP8 && c >= CPK / 2) return (2 * t) & SWZ;
    return t & SWZ;
  }
  // LDS chunk position of chunk c of key t (an involution within the key row)
  __device__ static int chunk_pos(int t, int c) { return t * CPK + (c ^ swz(t, c)); }
  static constexpr int TILE_BYTES = 16 * RB;
  static constexpr int IPT = TILE_BYTES / 1024;     // 1 KiB direct-to-LDS loads per tile
};

struct TileInfo {
  const char* kp;  // byte address of slot 0 of the tile, head kvh, in K
  const char* vp;  // same in V
  int nvalid;      // slots [0, nvalid) hold visible keys (1..16)
  float bias;      // log2-domain logit bias of the tile (segment partials: 0)
  int key0;        // key index of slot 0 (restricted numbering; paged modes);
                   // fused segments: position of slot 0 among the query's live keys
  int g0;          // fused segments: segment holding slot 0
};

// Causal query block (paged): row r of a tile sees keys [lo, hi] of the
// restricted numbering, hi = L' - sq + t(r), lo = hi - window_left (no lower
// bound without a window).  `on` is false for tiles every row sees whole.
struct RowMask {
  bool on;
  int hi, lo;
};

// Copy of a wave-uniform 64-bit value in scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint64_t a = (uint64_t)x;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// K/V bytes are read exactly once per launch: non-temporal loads keep them
// from displacing anything in the caches (measured +14% on random 8 KiB pages).
__device__ __forceinline__ u32x4 stream_load16(const char* src) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
}

template <int VDW>
__device__ __forceinline__ void load_v(uint32_t (&dst)[VDW], const char* src) {
  if constexpr (VDW == 4) {
    const u32x4 x = stream_load16(src);
    dst[0] = x[0]; dst[1] = x[1]; dst[2] = x[2]; dst[3] = x[3];
  } else if constexpr (VDW == 2) {
    const u32x2 x = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(src));
    dst[0] = x[0]; dst[1] = x[1];
  } else {
    dst[0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(src));
  }
}

template <int VDW>
__device__ __forceinline__ void lds_read_v(uint32_t (&dst)[VDW], const char* src) {
  if constexpr (VDW == 4) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(src);
    dst[0] = x[0]; dst[1] = x[1]; dst[2] = x[2]; dst[3] = x[3];
  } else if constexpr (VDW == 2) {
    const u32x2 x = *reinterpret_cast<const u32x2*>(src);
    dst[0] = x[0]; dst[1] = x[1];
  } else {
    dst[0] = *reinterpret_cast<const uint32_t*>(src);
  }
}

// Raw K/V bytes of one tile as one lane holds them: K pieces of key l%16 and
// the V values of keys 4*(l/16)+i.
template <int D, int KV>
struct Raw {
  u32x4 k[Geo<D, KV>::KLD];
  uint32_t v[4][Geo<D, KV>::VDW];
};

// MFMA operands of one tile: K in the query's S^T operand type, V^T in the
// P.V type (the query's 16-bit type; bf16 for an fp8 query).
template <int D, int QT>
struct Frags {
  typename QTypes<QT>::QOp kf[D / 32];
  u32x2 vA[D / 16];
};

// S^T operand K from the raw K pieces of one lane (key l%16; piece i holds
// stored bytes 64i + 16*(l/16) .. +15 of the key row).
template <int D, int KV, int QT>
__device__ __forceinline__ void k_operands(const u32x4 (&rk)[Geo<D, KV>::KLD], Frags<D, QT>& f) {
  using G = Geo<D, KV>;
  if constexpr (QT == K_FP8) {
    static_assert(KV == K_FP8, "an fp8 query needs an fp8 cache");
    // the stored bytes are the fp8 operand
#pragma unroll
    for (int c2 = 0; c2 < G::KLD; ++c2) {
      f.kf[2 * c2] = u32x2{rk[c2][0], rk[c2][1]};
      f.kf[2 * c2 + 1] = u32x2{rk[c2][2], rk[c2][3]};
    }
  } else if constexpr (KV == K_FP8) {
#pragma unroll
    for (int c2 = 0; c2 < G::KLD; ++c2) {
      uint32_t a0, a1, a2, a3, b0, b1, b2, b3;
      fp8x4_to_16<QT>(rk[c2][0], a0, a1);
      fp8x4_to_16<QT>(rk[c2][1], a2, a3);
      fp8x4_to_16<QT>(rk[c2][2], b0, b1);
      fp8x4_to_16<QT>(rk[c2][3], b2, b3);
      f.kf[2 * c2] = u32x4{a0, a1, a2, a3};
      f.kf[2 * c2 + 1] = u32x4{b0, b1, b2, b3};
    }
  } else {
#pragma unroll
    for (int kc = 0; kc < G::NKC; ++kc) f.kf[kc] = rk[kc];
  }
}

template <int D, int KV, int QT>
__device__ __forceinline__ void make_frags(const Raw<D, KV>& r, Frags<D, QT>& f) {
  using G = Geo<D, KV>;
  constexpr int PV = QTypes<QT>::PV;
  k_operands<D, KV, QT>(r.k, f);
  uint32_t v16[4][G::VPL / 2];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (KV == K_FP8) {
#pragma unroll
      for (int w = 0; w < G::VDW; ++w) fp8x4_to_16<PV>(r.v[i][w], v16[i][2 * w], v16[i][2 * w + 1]);
    } else {
#pragma unroll
      for (int w = 0; w < G::VDW; ++w) v16[i][w] = r.v[i][w];
    }
  }
#pragma unroll
  for (int j = 0; j < G::VPL; ++j) {
    const int w = j >> 1;
    if ((j & 1) == 0)
      f.vA[j] = u32x2{lo_lo(v16[0][w], v16[1][w]), lo_lo(v16[2][w], v16[3][w])};
    else
      f.vA[j] = u32x2{hi_hi(v16[0][w], v16[1][w]), hi_hi(v16[2][w], v16[3][w])};
  }
}

// K/V of one 16-slot tile straight into registers (attn_kernel's layout):
// lane l loads the K pieces of key l%16 and the V values of keys 4*(l/16)+i.
// kb / vb: slot 0 of the tile in K and V; tsb: bytes between slots.  Slots at
// or past nvalid read slot 0 (inside the tile; masked out of S later).
// Where a key's V share is 8 bytes per lane (fp8 with D = 128, 16-bit with
// D = 64), V arrives as two 16-byte loads per lane instead of four 8-byte ones
// (fewer load instructions per tile: fp8 Split-KV decode 358 -> 347 us): the
// lane pair (2m, 2m+1) loads head dims 16m .. 16m+15 of keys 4*(l/16) + {0, 1}
// (even lane) and {2, 3} (odd lane), and pair_v_regs swaps halves before use.
template <int D, int KV>
__device__ __forceinline__ void load_tile_regs(Raw<D, KV>& r, const char* kb, const char* vb,
                                               uint32_t tsb, int nvalid, int g4, int c16) {
  using G = Geo<D, KV>;
  const uint32_t ks = c16 < nvalid ? c16 : 0;
  const uint32_t koff = ks * tsb + 16 * g4;
#pragma unroll
  for (int i = 0; i < G::KLD; ++i) r.k[i] = stream_load16(kb + (koff + 64 * i));
  if constexpr (G::VDW == 2) {
    const int h = c16 & 1;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int key = 4 * g4 + 2 * h + i;
      const uint32_t vs = key < nvalid ? key : 0;
      const u32x4 x = stream_load16(vb + (vs * tsb + 16 * (c16 >> 1)));
      r.v[2 * i][0] = x[0];
      r.v[2 * i][1] = x[1];
      r.v[2 * i + 1][0] = x[2];
      r.v[2 * i + 1][1] = x[3];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t vs = 4 * g4 + i < nvalid ? 4 * g4 + i : 0;
      load_v<G::VDW>(r.v[i], vb + (vs * tsb + G::VB * c16));
    }
  }
}

// Lane-pair exchange after 16-byte V loads (see load_tile_regs): afterwards
// r.v[i] holds head dims 8*(l%16) .. +7 of key 4*(l/16) + i, as 8-byte loads
// would deliver them.
template <int D, int KV>
__device__ __forceinline__ void pair_v_regs(Raw<D, KV>& r, int c16) {
  const bool odd = (c16 & 1) != 0;
  uint32_t keep[2][2], send[2][2], recv[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      keep[i][w] = odd ? r.v[2 * i + 1][w] : r.v[2 * i][w];
      send[i][w] = odd ? r.v[2 * i][w] : r.v[2 * i + 1][w];
      // quad_perm(1, 0, 3, 2): lanes 2m and 2m+1 swap
      recv[i][w] = (uint32_t)__builtin_amdgcn_mov_dpp((int)send[i][w], 0xB1, 0xF, 0xF, false);
    }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      r.v[i][w] = odd ? recv[i][w] : keep[i][w];
      r.v[2 + i][w] = odd ? keep[i][w] : recv[i][w];
    }
}

// Query fragments (B operand of S^T = K Q^T) for row tile starting at `row0`:
// the same head dims per lane and register as the K operand of make_frags.
template <int D, int KV, int QT>
__device__ __forceinline__ void load_q(typename QTypes<QT>::QOp (&qf)[D / 32], const void* q,
                                       int row0, int R, int G, int kvh, int qb, int sq, int Hq,
                                       int g4, int c16) {
  using QOp = typename QTypes<QT>::QOp;
  constexpr int EB = QT == K_FP8 ? 1 : 2;
  const int rr = row0 + c16;
  if (rr < R) {
    const int t = rr / G, gg = rr % G;
    const int h = kvh * G + gg;
    const char* qrow = static_cast<const char*>(q) + ((((int64_t)qb * sq + t) * Hq + h) * D) * EB;
#pragma unroll
    for (int kc = 0; kc < D / 32; ++kc) {
      const int d = (KV == K_FP8) ? 64 * (kc >> 1) + 16 * g4 + 8 * (kc & 1) : 32 * kc + 8 * g4;
      qf[kc] = *reinterpret_cast<const QOp*>(qrow + d * EB);
    }
  } else {
#pragma unroll
    for (int kc = 0; kc < D / 32; ++kc) qf[kc] = QOp{};
  }
}

// One 16-key tile against one 16-row tile: S^T, online softmax, O^T += V^T P^T.
// EMPTY_ROWS: a row may have seen only -inf logits so far (causal rows before
// their first key; fused segments whose bias is -inf), so its running max can
// still be -inf and the exponent reference must stay finite.
// KEY_BIAS: each of the lane's four keys carries its own bias (kbias[i] for key
// 4*g4 + i: a tile packed from several segments); otherwise every key of the
// tile carries `bias`.
template <int D, int QT, bool CAUSAL = false, bool EMPTY_ROWS = CAUSAL, bool KEY_BIAS = false,
          typename Hook = NoHook, typename VHook = NoHook>
__device__ __forceinline__ void attend_tile(const Frags<D, QT>& f,
                                            const typename QTypes<QT>::QOp (&qf)[D / 32],
                                            f32x4 (&acc)[D / 16], float& m_run, float& l_run,
                                            float scale_log2, float bias, int nvalid, int g4,
                                            int key0 = 0, RowMask rm = RowMask{false, 0, 0},
                                            const Hook& mid = Hook{}, const VHook& vload = VHook{},
                                            f32x4 kbias = f32x4{0.f, 0.f, 0.f, 0.f}) {
  f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kc = 0; kc < D / 32; ++kc) sacc = qk_mfma<QT>(f.kf[kc], qf[kc], sacc);
  if constexpr (!std::is_same<Hook, NoHook>::value) {
    __builtin_amdgcn_sched_barrier(0);
    mid();
    __builtin_amdgcn_sched_barrier(0);
  }
  float s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = sacc[i] * scale_log2 + (KEY_BIAS ? kbias[i] : bias);
  if (nvalid < 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * g4 + i >= nvalid) s[i] = kNegInf;
  }
  if constexpr (CAUSAL) {
    if (rm.on) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = key0 + 4 * g4 + i;
        if (key > rm.hi || key < rm.lo) s[i] = kNegInf;
      }
    }
  }
  float tmax = vmax(vmax(s[0], s[1]), vmax(s[2], s[3]));
  tmax = max_across_groups(tmax);
  // Lazy rescale: the reference max m_run only moves when some row of the
  // wave sees a logit more than kRescaleSlack above it, so p = 2^(s - m_run)
  // stays <= 2^kRescaleSlack and the O / l rescale is skipped on most tiles.
  // Softmax does not depend on the reference, only on it bounding the terms.
  if (__ballot(tmax > m_run + kRescaleSlack) != 0) {
    const float m_new = vmax(m_run, tmax);
    float alpha = fast_exp2(m_run - m_new);  // 0 on the first tile (m_run = -inf)
    // a row that has seen no finite logit yet (m_new = -inf) keeps its zeros
    if constexpr (EMPTY_ROWS) alpha = m_new == kNegInf ? 1.f : alpha;
    l_run *= alpha;
#pragma unroll
    for (int j = 0; j < D / 16; ++j) acc[j] *= alpha;
    m_run = m_new;
  }
  // rows with no finite logit so far have only -inf logits: any finite reference
  float m_ref = m_run;
  if constexpr (EMPTY_ROWS) m_ref = m_run == kNegInf ? 0.f : m_run;
  float pr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(s[i] - m_ref);
  l_run += (pr[0] + pr[1]) + (pr[2] + pr[3]);
  constexpr int PV = QTypes<QT>::PV;
  const u32x2 pB = u32x2{pack2<PV>(pr[0], pr[1]), pack2<PV>(pr[2], pr[3])};
  if constexpr (!std::is_same<VHook, NoHook>::value) {
    __builtin_amdgcn_sched_barrier(0);
    vload();  // V^T operands read only now: fewer registers live across the softmax
  }
#pragma unroll
  for (int j = 0; j < D / 16; ++j) acc[j] = mfma_16x16x16<PV>(f.vA[j], pB, acc[j]);
}

// Two 16-key tiles (keys 0..15 in f0, 16..31 in f1) against one 16-row tile,
// with one softmax update and P.V on the 32-deep MFMA: its contraction index
// 8*(l/16) + j pairs keys 4*(l/16) + j of the first tile (j < 4) with keys
// 16 + 4*(l/16) + j - 4 of the second, so A and B are the two 16-key operands
// side by side.  Every row has a live key in the first tile (no causal mask).
template <int D, int QT, typename Hook, typename VHook, typename VOp>
__device__ __forceinline__ void attend_tile32(const Frags<D, QT>& f0, const Frags<D, QT>& f1,
                                              const typename QTypes<QT>::QOp (&qf)[D / 32],
                                              f32x4 (&acc)[D / 16], float& m_run, float& l_run,
                                              float scale_log2, int nvalid0, int nvalid1, int g4,
                                              const Hook& mid, const VHook& vload, const VOp& vop) {
  f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f}, sb = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kc = 0; kc < D / 32; ++kc) sa = qk_mfma<QT>(f0.kf[kc], qf[kc], sa);
#pragma unroll
  for (int kc = 0; kc < D / 32; ++kc) sb = qk_mfma<QT>(f1.kf[kc], qf[kc], sb);
  float s[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s[i] = sa[i] * scale_log2;
    s[4 + i] = sb[i] * scale_log2;
  }
  __builtin_amdgcn_sched_barrier(0);
  mid();
  __builtin_amdgcn_sched_barrier(0);
  if (nvalid0 < 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * g4 + i >= nvalid0) s[i] = kNegInf;
  }
  if (nvalid1 < 16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * g4 + i >= nvalid1) s[4 + i] = kNegInf;
  }
  float tmax = vmax(vmax(vmax(s[0], s[1]), vmax(s[2], s[3])), vmax(vmax(s[4], s[5]), vmax(s[6], s[7])));
  tmax = max_across_groups(tmax);
  if (__ballot(tmax > m_run + kRescaleSlack) != 0) {
    const float m_new = vmax(m_run, tmax);
    const float alpha = fast_exp2(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int j = 0; j < D / 16; ++j) acc[j] *= alpha;
    m_run = m_new;
  }
  float pr[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) pr[i] = fast_exp2(s[i] - m_run);
  l_run += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
  constexpr int PV = QTypes<QT>::PV;
  const u32x4 pB = u32x4{pack2<PV>(pr[0], pr[1]), pack2<PV>(pr[2], pr[3]), pack2<PV>(pr[4], pr[5]),
                         pack2<PV>(pr[6], pr[7])};
  __builtin_amdgcn_sched_barrier(0);
  vload();
#pragma unroll
  for (int j = 0; j < D / 16; ++j) acc[j] = mfma_16x16x32<PV>(vop(j), pB, acc[j]);
}

// Write one lane's part of a finished 16-row tile: row row0 + l%16, values
// acc[j][i] / l (times v_scale) at head dim
//   interleaved layout (BLOCKED = false):  VPL*(4*(l/16)+i) + j
//   blocked layout     (BLOCKED = true):   16*j + 4*(l/16) + i
// Partial outputs (fp32) of rows that saw no key are skipped; their LSE is -inf.
template <int D, bool BLOCKED = false>
__device__ __forceinline__ void store_tile(const f32x4 (&acc)[D / 16], float m_run, float l_run,
                                           float v_scale, void* out, int out_kind, float* lse,
                                           int64_t orow, bool partial, int g4) {
  constexpr int VPL = D / 16;
  const bool live = l_run > 0.f;
  const float inv = live ? v_scale / l_run : 0.f;
  if (live || !partial) {
    if constexpr (BLOCKED) {
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        const float vals[4] = {acc[j][0] * inv, acc[j][1] * inv, acc[j][2] * inv, acc[j][3] * inv};
        store_row<4>(out, orow * D + 16 * j + 4 * g4, out_kind, vals);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float vals[VPL];
#pragma unroll
        for (int j = 0; j < VPL; ++j) vals[j] = acc[j][i] * inv;
        store_row<VPL>(out, orow * D + VPL * (4 * g4 + i), out_kind, vals);
      }
    }
  }
  if (g4 == 0 && lse) lse[orow] = live ? (m_run + log2f(l_run)) * kLn2 : kNegInf;
}

// Pages / tiles of one (request, split) of the paged mode.
struct PagedRange {
  SeqView sv;
  SplitRange sr;
  int TPP;      // 16-slot tiles per page
  int tok_end;  // first invisible key of the split (restricted numbering)
  int n_tiles;
};

__device__ __forceinline__ PagedRange paged_range(const AttnParams& p, int item, int split) {
  PagedRange r;
  r.sv = seq_view(p.seq_lens[item], p.window, p.sq, p.P, p.bt_width);
  r.sr = split_range(r.sv, p.P, p.S, p.chunk, split);
  r.TPP = (p.P + 15) >> 4;
  r.tok_end = r.sr.tok0 + r.sr.n_tok;
  r.n_tiles = 0;
  if (r.sr.n_pages > 0) {
    const int last_count = r.sr.n_tok - (r.sr.n_pages - 1) * p.P;
    r.n_tiles = (r.sr.n_pages - 1) * r.TPP + ((last_count + 15) >> 4);
  }
  return r;
}

// Tile `it` of a paged split: page, first slot and number of visible slots.
__device__ __forceinline__ void paged_tile(const AttnParams& p, const PagedRange& r, int it,
                                           int& page, int& slot0, int& nvalid) {
  const int pin = r.TPP == 1 ? it : it / r.TPP;  // pages of up to 16 slots: no division
  const int u = it - pin * r.TPP;
  page = r.sr.first_page + pin;
  slot0 = 16 * u;
  const int tok0 = page * p.P + slot0;
  int nv = p.P - slot0;
  if (nv > 16) nv = 16;
  if (r.tok_end - tok0 < nv) nv = r.tok_end - tok0;
  nvalid = nv;
}

// Wait until this wave's loads of the current tile have landed, i.e. until at
// most `ahead` later tiles (IPW loads each) are still in flight.  s_waitcnt
// takes an immediate, hence the unrolled chain.
template <int IPW, int A>
__device__ __forceinline__ void wait_tiles_ahead(int ahead) {
  static_assert(A * IPW <= 63, "vmcnt holds at most 63 outstanding loads");
  if constexpr (A <= 0) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  } else {
    if (ahead >= A) __builtin_amdgcn_s_waitcnt(vmcnt_imm(A * IPW));
    else wait_tiles_ahead<IPW, A - 1>(ahead);
  }
}

// f(integral_constant<S>) for S = B .. E-1 in order while it returns true
// (compile-time stage numbers for the unrolled ring loop).
template <int B, int E, typename F>
__device__ __forceinline__ bool static_all(F&& f) {
  if constexpr (B < E) {
    if (!f(std::integral_constant<int, B>{})) return false;
    return static_all<B + 1, E>(f);
  } else {
    return true;
  }
}

// Longest-first dispatch: the request with the given rank when requests are
// ordered by decreasing visible length (ties by index).  Work items are laid
// out rank-major, so the hardware starts the longest requests' workgroups
// first and the short ones fill the tail.  Every wave of the workgroup
// computes it (one 64-wide load and a 64-step compare).  Used for up to 64
// requests; larger batches keep their natural order.
__device__ __forceinline__ int request_of_rank(const AttnParams& p, int rank) {
  if (p.items > 64) return rank;
  const int lane = threadIdx.x & 63;
  int len = -1;
  if (lane < p.items) len = seq_view(p.seq_lens[lane], p.window, p.sq, p.P, p.bt_width).len;
  int r = 0;
  for (int j = 0; j < p.items; ++j) {
    const int lj = __builtin_amdgcn_readlane(len, j);
    r += (lj > len) | ((lj == len) & (j < lane));
  }
  const uint64_t hit = __ballot(lane < p.items && r == rank);
  return (int)__builtin_ctzll(hit);
}

// Pool page of restricted page `page`, clamped into the pool.
__device__ __forceinline__ int32_t load_phys(const AttnParams& p, const int32_t* trow,
                                             const SeqView& sv, int page) {
  int32_t ph = trow[table_column(sv, page, p.bt_width)];
  return ph < 0 ? 0 : (ph >= p.num_pages ? p.num_pages - 1 : ph);
}

// Fused segments of query n (dash_attention page, flash_dash_attention): lane
// g <= topk describes segment g (the topk remote segments, then the local
// one).  The query's live keys are numbered in segment order, so live key j
// of segment g is key cum_start + j and sits at row j + adj of the query.
struct SegLanes {
  int cum_end = 0x7fffffff;    // live keys of segments 0..g
  int cum_start = 0x7fffffff;  // live keys before segment g
  int adj = 0;                 // segment g's first row minus cum_start
  float bias = 0.f;            // segment bias in log2 units (local segment: 0)
  int n_keys = 0;              // live keys of the query (every lane)
};

__device__ __forceinline__ SegLanes seg_lanes(const AttnParams& p, int n, int lane) {
  SegLanes s;
  const int Gs = p.topk + 1;
  int u = 0;
  if (lane < Gs) {
    const int cap = lane < p.topk ? p.bs : p.local;
    u = p.used[(int64_t)n * Gs + lane];
    u = u < 0 ? 0 : (u > cap ? cap : u);
    s.bias = lane < p.topk ? p.bias[(int64_t)n * p.topk + lane] * kLog2e : 0.f;
  }
  int cum = u;  // inclusive prefix sum of live keys across lanes
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(cum, off, 64);
    if (lane >= off) cum += o;
  }
  s.n_keys = __builtin_amdgcn_readlane(cum, 63);  // a scalar: tile loops stay uniform
  if (lane < Gs) {
    s.cum_end = cum;
    s.cum_start = cum - u;
    s.adj = (lane < p.topk ? lane * p.bs : p.topk * p.bs) - s.cum_start;
  }
  return s;
}

// Segment holding live key `key` (wave-uniform key).
__device__ __forceinline__ int seg_of_key(const SegLanes& s, int key) {
  return __builtin_amdgcn_readfirstlane(__builtin_popcountll(__ballot(s.cum_end <= key)));
}

// Per-lane `field` (held by lane g for segment g) of the segment holding each
// of the lane's keys key0 + d[j], d[j] < 16, where g0 holds key0.  Only the
// segments that start inside the tile are visited: a wave-uniform loop,
// usually 0-2 rounds.
template <int N>
__device__ __forceinline__ void seg_field(const SegLanes& s, int topk, int key0, int g0,
                                          const int (&d)[N], int field, int (&out)[N]) {
  const int v0 = __builtin_amdgcn_readlane(field, g0);
#pragma unroll
  for (int j = 0; j < N; ++j) out[j] = v0;
  for (int g = g0 + 1; g <= topk; ++g) {
    const int thr = __builtin_amdgcn_readlane(s.cum_start, g) - key0;
    if (thr >= 16) break;
    const int vg = __builtin_amdgcn_readlane(field, g);
#pragma unroll
    for (int j = 0; j < N; ++j) out[j] = d[j] >= thr ? vg : out[j];
  }
}

}  // namespace

// ================================================================================
// attn_kernel: waves split the keys of a work item.
//   paged:          work item (request, kv head, row group, split)
//   segment:        (query, segment, kv head, row group)
//   segment fused:  (query, kv head, row group); segment g's logits get its bias
// CAUSAL (paged only): bottom-right causal rows with an exact per-token window.
// ================================================================================
template <int D, int RT, int NW, int KV, int QT, int MODE, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void attn_kernel(const AttnParams p) {
  using G = Geo<D, KV>;
  constexpr int KB = G::KB;
  constexpr int VPL = G::VPL;
  constexpr int ROWS = RT * 16;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int g4 = lane >> 4;
  const int c16 = lane & 15;

  uint32_t bid = blockIdx.x;  // 32-bit: the grid never exceeds 2^31 workgroups
  int split = 0;
  if constexpr (MODE == MODE_PAGED) {
    split = (int)(bid % (uint32_t)p.S);
    bid /= (uint32_t)p.S;
  }
  const int rg = (int)(bid % (uint32_t)p.RG);
  bid /= (uint32_t)p.RG;
  const int kvh = (int)(bid % (uint32_t)p.Hkv);
  int item = (int)(bid / (uint32_t)p.Hkv);
  if constexpr (MODE == MODE_PAGED) item = request_of_rank(p, item);

  const int64_t ts_b = p.token_stride * KB;
  const int64_t head_off_b = (int64_t)kvh * p.head_stride * KB;

  int n_tiles = 0;
  int qb = item;  // query row block
  PagedRange pr{};
  int64_t seg_tok0 = 0;
  int seg_used = 0;
  // fused segments: the live keys of the query's segments are numbered in
  // segment order and cut into 16-key tiles, so a tile may span segments (only
  // the query's last tile is partly filled)
  SegLanes sl;
  int64_t f_qoff_b = 0;  // byte offset of the query's first row, at this kv head

  if constexpr (MODE == MODE_PAGED) {
    pr = paged_range(p, item, split);
    n_tiles = pr.n_tiles;
  } else if constexpr (MODE == MODE_SEGMENT) {
    const int Gs = p.topk + 1;
    const int n = item / Gs, gs = item % Gs;
    const int cap = gs < p.topk ? p.bs : p.local;
    int u = p.used[item];
    u = u < 0 ? 0 : (u > cap ? cap : u);
    seg_used = u;
    seg_tok0 = (int64_t)n * (p.topk * p.bs + p.local) + (gs < p.topk ? gs * p.bs : p.topk * p.bs);
    n_tiles = (u + 15) >> 4;
    qb = n;
  } else {
    const int n = item;
    sl = seg_lanes(p, n, lane);
    n_tiles = (sl.n_keys + 15) >> 4;
    f_qoff_b = (int64_t)n * (p.topk * p.bs + p.local) * ts_b + head_off_b;
    qb = n;
  }

  const int row_base = rg * ROWS;
  typename QTypes<QT>::QOp qf[RT][D / 32];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
    load_q<D, KV, QT>(qf[rt], p.q, row_base + rt * 16, p.R, p.G, kvh, qb, p.sq, p.Hq, g4, c16);

  // paged: lane i caches the pool page of the wave's tile k0 + i
  int32_t phys_vec = 0;
  int k0 = -64;
  const int32_t* trow = nullptr;
  if constexpr (MODE == MODE_PAGED) trow = p.block_table + (int64_t)item * p.bt_stride;

  auto tile_info = [&](int k) -> TileInfo {
    const int it = wave + NW * k;
    TileInfo ti;
    ti.bias = 0.f;
    ti.key0 = 0;
    ti.g0 = 0;
    if constexpr (MODE == MODE_PAGED) {
      if (k - k0 >= 64) {
        k0 = k;
        const int itl = wave + NW * (k0 + lane);
        int32_t ph = 0;
        if (itl < n_tiles)
          ph = load_phys(p, trow, pr.sv, pr.sr.first_page + (pr.TPP == 1 ? itl : itl / pr.TPP));
        phys_vec = ph;
      }
      const int32_t phys = __builtin_amdgcn_readlane(phys_vec, k - k0);
      int page, slot0, nv;
      paged_tile(p, pr, it, page, slot0, nv);
      ti.nvalid = nv;
      ti.key0 = page * p.P + slot0;
      const int64_t off = ((int64_t)phys * p.page_stride + (int64_t)slot0 * p.token_stride) * KB + head_off_b;
      ti.kp = p.k + off;
      ti.vp = p.v + off;
    } else if constexpr (MODE == MODE_SEGMENT) {
      const int64_t tok = seg_tok0 + 16 * it;
      const int nv = seg_used - 16 * it;
      ti.nvalid = nv > 16 ? 16 : nv;
      const int64_t off = tok * ts_b + head_off_b;
      ti.kp = p.k + off;
      ti.vp = p.v + off;
    } else {
      // live keys 16*it .. 16*it+15; slot 0 lies in the first segment that
      // ends after it (segments are found per key when the tile is loaded)
      ti.key0 = 16 * it;
      ti.g0 = seg_of_key(sl, ti.key0);
      const int nv = sl.n_keys - ti.key0;
      ti.nvalid = nv > 16 ? 16 : nv;
      ti.kp = p.k + f_qoff_b;
      ti.vp = p.v + f_qoff_b;
    }
    return ti;
  };

  // Tile bases are wave-uniform (scalar registers); lanes add 32-bit offsets,
  // so each load is a scalar base plus one VGPR offset.
  const uint32_t tsb = (uint32_t)ts_b;  // 16 * tsb < 2^31 (checked at the boundary)
  constexpr bool kPairV = G::VDW == 2;
  auto load_tile = [&](Raw<D, KV>& r, const TileInfo& ti) {
    if constexpr (MODE != MODE_SEGMENT_FUSED) {
      // offsets from the kernel-argument pointers keep the global address space
      load_tile_regs<D, KV>(r, p.k + uniform64(ti.kp - p.k), p.k + uniform64(ti.vp - p.k), tsb,
                            ti.nvalid, g4, c16);
    } else {
      // key slots: K of key c16, V of keys 4*g4 + i (slots past the live keys read key 0)
      int d[5], row[5];
      d[0] = c16 < ti.nvalid ? c16 : 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) d[1 + i] = 4 * g4 + i < ti.nvalid ? 4 * g4 + i : 0;
      seg_field(sl, p.topk, ti.key0, ti.g0, d, sl.adj, row);
#pragma unroll
      for (int j = 0; j < 5; ++j) row[j] += ti.key0 + d[j];
      const char* kq = p.k + uniform64(ti.kp - p.k);
      const char* vq = p.k + uniform64(ti.vp - p.k);
      const uint64_t koff = (uint64_t)(uint32_t)row[0] * tsb + 16 * g4;
#pragma unroll
      for (int i = 0; i < G::KLD; ++i) r.k[i] = stream_load16(kq + (koff + 64 * i));
      if constexpr (G::VDW == 2) {
        // as load_tile_regs: the lane pair (2m, 2m+1) loads keys 4*g4 + {0, 1} / {2, 3}
        const bool h = (c16 & 1) != 0;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int rw = h ? row[3 + i] : row[1 + i];
          const u32x4 x = stream_load16(vq + ((uint64_t)(uint32_t)rw * tsb + 16 * (c16 >> 1)));
          r.v[2 * i][0] = x[0];
          r.v[2 * i][1] = x[1];
          r.v[2 * i + 1][0] = x[2];
          r.v[2 * i + 1][1] = x[3];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          load_v<G::VDW>(r.v[i], vq + ((uint64_t)(uint32_t)row[1 + i] * tsb + G::VB * c16));
      }
    }
  };
  auto pair_v = [&](Raw<D, KV>& r) { pair_v_regs<D, KV>(r, c16); };

  f32x4 acc[RT][VPL];
  float m_run[RT], l_run[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = kNegInf;
    l_run[rt] = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) acc[rt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // causal bounds of this lane's rows; tiles inside [lo_max, hi_min] need no mask
  int row_hi[RT] = {}, row_lo[RT] = {};
  int hi_min = 0, lo_max = 0;
  if constexpr (CAUSAL) {
    const int Lr = pr.sv.len;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int t = (row_base + rt * 16 + c16) / p.G;
      row_hi[rt] = Lr - p.sq + t;
      row_lo[rt] = p.window_left >= 0 ? row_hi[rt] - p.window_left : INT32_MIN;
    }
    hi_min = Lr - p.sq;
    lo_max = p.window_left >= 0 ? Lr - 1 - p.window_left : INT32_MIN;
  }
  auto attend = [&](const Frags<D, QT>& f, const TileInfo& ti) {
    const bool on = CAUSAL && (ti.key0 + 15 > hi_min || ti.key0 < lo_max);
    f32x4 kbias = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (MODE == MODE_SEGMENT_FUSED) {
      // bias of the segment of each of the lane's keys 4*g4 + i (the S^T layout)
      int d[5], b[5];
      d[0] = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) d[1 + i] = 4 * g4 + i;
      seg_field(sl, p.topk, ti.key0, ti.g0, d, __float_as_int(sl.bias), b);
#pragma unroll
      for (int i = 0; i < 4; ++i) kbias[i] = __int_as_float(b[1 + i]);
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
      attend_tile<D, QT, CAUSAL, CAUSAL || MODE == MODE_SEGMENT_FUSED, MODE == MODE_SEGMENT_FUSED>(
          f, qf[rt], acc[rt], m_run[rt], l_run[rt], p.qk_scale_log2, ti.bias, ti.nvalid, g4,
          ti.key0, RowMask{on, row_hi[rt], row_lo[rt]}, NoHook{}, NoHook{}, kbias);
  };

  // main loop: tile k+1 is in flight while tile k is computed
  if (wave < n_tiles) {
    TileInfo ti = tile_info(0);
    Raw<D, KV> cur;
    load_tile(cur, ti);
    for (int k = 0;; ++k) {
      const bool more = wave + NW * (k + 1) < n_tiles;
      TileInfo tn = ti;
      Raw<D, KV> nxt;
      if (more) {
        tn = tile_info(k + 1);
        load_tile(nxt, tn);
      }
      Frags<D, QT> f;
      if constexpr (kPairV) pair_v(cur);
      make_frags<D, KV, QT>(cur, f);
      attend(f, ti);
      if (!more) break;
      cur = nxt;
      ti = tn;
    }
  }

#pragma unroll
  for (int rt = 0; rt < RT; ++rt) l_run[rt] = sum_across_groups(l_run[rt]);

  // ---- epilogue ----------------------------------------------------------------
  auto out_row = [&](int rr) -> int64_t {
    const int t = rr / p.G, gg = rr % p.G;
    const int h = kvh * p.G + gg;
    if constexpr (MODE == MODE_SEGMENT) return (int64_t)item * p.Hq + h;
    return ((int64_t)qb * p.sq + t) * p.Hq + h;
  };
  float* lse_base = p.lse;
  void* o_base = p.out;
  if (p.partial && MODE == MODE_PAGED) {
    lse_base = p.lse + (int64_t)split * p.split_stride_lse;
    o_base = reinterpret_cast<float*>(p.out) + (int64_t)split * p.split_stride_o;
  }

  if constexpr (NW == 1) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int rr = row_base + rt * 16 + c16;
      if (rr < p.R)
        store_tile<D>(acc[rt], m_run[rt], l_run[rt], p.v_scale, o_base, p.out_kind, lse_base,
                      out_row(rr), p.partial, g4);
    }
  } else {
    // merge buffer in dynamic LDS, sized by the rows that exist: rows of this
    // workgroup at or past p.R are never written or read
    extern __shared__ float merge_lds[];
    const int rows_held = merge_rows(p.R, ROWS);
    constexpr int OS = D + 4;  // padded row stride
    float* red_o = merge_lds;                          // [NW][rows_held][OS]
    float* red_m = merge_lds + NW * rows_held * OS;    // [NW][rows_held]
    float* red_l = red_m + NW * rows_held;             // [NW][rows_held]
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int row = rt * 16 + c16;
      if (row < rows_held) {
        float* dst = red_o + (wave * rows_held + row) * OS;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < VPL; ++j) dst[VPL * (4 * g4 + i) + j] = acc[rt][j][i];
        if (g4 == 0) {
          red_m[wave * rows_held + row] = m_run[rt];
          red_l[wave * rows_held + row] = l_run[rt];
        }
      }
    }
    __syncthreads();
    constexpr int QD = D / 4;
    for (int e = threadIdx.x; e < rows_held * QD; e += NW * 64) {
      const int row = e / QD;
      const int dq = (e - row * QD) * 4;
      const int rr = row_base + row;
      if (rr >= p.R) continue;
      const int64_t orow = out_row(rr);
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = vmax(M, red_m[w * rows_held + row]);
      float o[4] = {0.f, 0.f, 0.f, 0.f};
      float tot = 0.f;
      if (M != kNegInf) {
        float wgt[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          wgt[w] = fast_exp2(red_m[w * rows_held + row] - M);
          tot += wgt[w] * red_l[w * rows_held + row];
        }
        const float inv = p.v_scale / tot;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const float c = wgt[w] * inv;
          const float* src = red_o + (w * rows_held + row) * OS + dq;
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] += c * src[q];
        }
      }
      const bool live = tot > 0.f;
      if (live || !p.partial) store_row<4>(o_base, orow * D + dq, p.out_kind, o);
      if (dq == 0 && lse_base) lse_base[orow] = live ? (M + log2f(tot)) * kLn2 : kNegInf;
    }
  }
}

// ================================================================================
// attn_shared_kernel (paged): work item (request, kv head, row group, split);
// wave w owns rows row_base + 16w .. +16, every wave attends every tile.
//
// LDS ring: stage s holds one tile as 16 keys x CPK 16-byte chunks, K chunks
// first then V chunks of each key, chunk c of key t stored at position
// Geo::chunk_pos(t, c) = t*CPK + (c ^ Geo::swz(t, c)).  The XOR keeps the
// K-operand reads (16 keys, same chunk) and the transposing V reads (two
// adjacent chunks of 4 keys per 16-lane group) on distinct banks (no
// conflicts with 32 or with 64 four-byte banks); direct-to-LDS loads write
// lane i's 16 bytes to position 64*j + i of instruction j, so each lane simply
// fetches the chunk that belongs at its position.  Instruction j of a tile is
// issued by wave j / (IPT / NW).
// ================================================================================
// Occupancy floor for the four- and eight-wave kernels: five waves per SIMD
// (96 VGPRs) with 16-bit queries, six (80) with fp8 queries.  The causal bf16
// kernel needs it to reach five without spilling; the two-wave kernels spill
// under it and keep the default.
template <int NW, int QT>
constexpr int kSharedMinWaves = NW >= 4 ? (QT == K_FP8 ? 6 : 5) : 1;

// KT: keys per staged tile.  The dense fp8-query block stages 32 keys (two
// 16-key sub-tiles, each from its own page slot range) and runs attend_tile32:
// one softmax update and half as many P.V MFMAs per key at the full 32-deep
// rate, for five instead of six waves per SIMD (84 VGPRs).
template <int D, int NW, int KV, int QT, int NBUF, bool CAUSAL, int KT = 16>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(KT == 32 ? 5 : kSharedMinWaves<NW, QT>)))
void attn_shared_kernel(const AttnParams p) {
  using G = Geo<D, KV>;
  constexpr int KB = G::KB;
  constexpr int VPL = G::VPL;
  static_assert(KT == 16 || (KT == 32 && !CAUSAL), "32-key tiles without the causal mask");
  constexpr int TB = G::TILE_BYTES * (KT / 16);  // bytes of a staged tile
  constexpr int IPW = TB / 1024 / NW;  // direct-to-LDS loads per wave per tile
  static_assert((TB / 1024) % NW == 0 && IPW >= 1, "tile loads must split evenly over the waves");
  static_assert(NBUF >= 2 && NBUF <= 8, "ring depth");
  // One LDS object per ring stage, addressed with compile-time stage numbers
  // (the tile loop is unrolled NBUF times).  The compiler can then tell that
  // reading stage s does not depend on the direct-to-LDS loads still landing
  // in the other stages; with a single array it waits for all of them first.
  __shared__ __attribute__((aligned(1024))) char ring0[TB];
  __shared__ __attribute__((aligned(1024))) char ring1[TB];
  __shared__ __attribute__((aligned(1024))) char ring2[NBUF > 2 ? TB : 16];
  __shared__ __attribute__((aligned(1024))) char ring3[NBUF > 3 ? TB : 16];
  __shared__ __attribute__((aligned(1024))) char ring4[NBUF > 4 ? TB : 16];
  __shared__ __attribute__((aligned(1024))) char ring5[NBUF > 5 ? TB : 16];
  __shared__ __attribute__((aligned(1024))) char ring6[NBUF > 6 ? TB : 16];
  __shared__ __attribute__((aligned(1024))) char ring7[NBUF > 7 ? TB : 16];
  auto stage_buf = [&](auto sc) -> char* {
    constexpr int s = decltype(sc)::value;
    if constexpr (s == 0) return ring0;
    else if constexpr (s == 1) return ring1;
    else if constexpr (s == 2) return ring2;
    else if constexpr (s == 3) return ring3;
    else if constexpr (s == 4) return ring4;
    else if constexpr (s == 5) return ring5;
    else if constexpr (s == 6) return ring6;
    else return ring7;
  };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int g4 = lane >> 4;
  const int c16 = lane & 15;

  uint32_t bid = blockIdx.x;
  const int split = (int)(bid % (uint32_t)p.S);
  bid /= (uint32_t)p.S;
  const int rg = (int)(bid % (uint32_t)p.RG);
  bid /= (uint32_t)p.RG;
  const int kvh = (int)(bid % (uint32_t)p.Hkv);
  const int item = request_of_rank(p, (int)(bid / (uint32_t)p.Hkv));

  const int64_t ts_b = p.token_stride * KB;
  const int64_t head_off_b = (int64_t)kvh * p.head_stride * KB;
  const PagedRange pr = paged_range(p, item, split);
  const int n_tiles = KT == 32 ? (pr.n_tiles + 1) >> 1 : pr.n_tiles;  // 16-key sub-tiles paired
  const int row0 = rg * (NW * 16) + wave * 16;

  typename QTypes<QT>::QOp qf[D / 32];
  load_q<D, KV, QT>(qf, p.q, row0, p.R, p.G, kvh, item, p.sq, p.Hq, g4, c16);

  // Pool pages, 64 tiles at a time: lane i of phys_vec holds the page of tile
  // k0 + i.  Lanes past the last tile read a valid (clamped) column that is
  // never used; entries are clamped into the pool where they are used.
  const int32_t* trow = p.block_table + (int64_t)item * p.bt_stride;
  auto table_batch = [&](int first) -> int32_t {
    const int kl = first + lane;
    // the divisor is passed through an opaque copy so its reciprocal is worked
    // out here, once per 64 tiles, instead of being held across the tile loop
    int tpp = pr.TPP;
    asm volatile("" : "+s"(tpp));
    return trow[table_column(pr.sv, pr.sr.first_page + (tpp == 1 ? kl : kl / tpp), p.bt_width)];
  };
  int32_t phys_vec = table_batch(0);
  int k0 = 0;
  // 32-key tiles: lane i holds the byte offset (pool page, clamped, and slot)
  // and the live slots of sub-tile k0 + i, worked out once per 64 sub-tiles,
  // so issuing a tile takes six v_readlane instead of a cursor walk, scalar
  // clamps and 64-bit multiplies (fp8-query block 3-4% faster)
  int64_t poff_vec = 0;
  int nv_vec = 0;
  auto sub_batch = [&](int first, int32_t ph) {
    ph = ph < 0 ? 0 : (ph >= p.num_pages ? p.num_pages - 1 : ph);
    const int j = first + lane;
    int tpp = pr.TPP;
    asm volatile("" : "+s"(tpp));
    const int pg = tpp == 1 ? j : j / tpp;
    const int u = j - pg * tpp;
    const int tok0 = (pr.sr.first_page + pg) * p.P + 16 * u;
    int nv = p.P - 16 * u;
    nv = nv > 16 ? 16 : nv;
    nv = pr.tok_end - tok0 < nv ? pr.tok_end - tok0 : nv;
    poff_vec = (int64_t)ph * (p.page_stride * KB) + (int64_t)(16 * u) * ts_b;
    nv_vec = nv;
  };
  if constexpr (KT == 32) sub_batch(0, phys_vec);

  // Lane-constant part of the source address of each chunk this wave copies:
  // instruction j = wave*IPW + u writes LDS position 64*j + lane, which holds
  // chunk c of key t (see the layout above).  Relative to K of slot 0 of a
  // tile; V chunks add the V - K distance.  `src0` is the same chunk of slot 0,
  // fetched instead when key t is past the end of a partial tile.
  const int64_t vk = p.v - p.k;
  int64_t src_slot0[IPW], src_key_off[IPW];
  int src_key[IPW], src_half[IPW];
#pragma unroll
  for (int u = 0; u < IPW; ++u) {
    const int pos = 64 * (wave * IPW + u) + lane;
    const int tt = pos / G::CPK;
    const int t = tt & 15;
    const int c = (pos % G::CPK) ^ G::swz(t, pos % G::CPK);  // chunk_pos is an involution per key
    src_slot0[u] = c < G::CPK / 2 ? 16 * c : vk + 16 * (c - G::CPK / 2);
    src_key_off[u] = t * ts_b;
    src_key[u] = t;
    src_half[u] = __builtin_amdgcn_readfirstlane(tt >> 4);  // one 16-key half per load
  }
  const int64_t page_b = p.page_stride * KB;
  const int TPP = pr.TPP;

  // Tile cursor: restricted page, sub-tile, first key (tiles are visited in order).
  struct Cursor {
    int page, u, tok0;
  };
  auto cursor_at0 = [&]() { return Cursor{pr.sr.first_page, 0, pr.sr.first_page * p.P}; };
  auto advance = [&](Cursor& c) {
    if (++c.u == TPP) {
      c.u = 0;
      ++c.page;
      c.tok0 = c.page * p.P;
    } else {
      c.tok0 += 16;
    }
  };
  auto cursor_valid = [&](const Cursor& c) {
    int nv = p.P - 16 * c.u;
    if (nv > 16) nv = 16;
    if (pr.tok_end - c.tok0 < nv) nv = pr.tok_end - c.tok0;
    return nv;
  };

  auto issue_tile = [&](int k, const Cursor& c, auto sc) {
    char* ring = stage_buf(sc);
    if constexpr (KT == 16) {
      if (k - k0 >= 64) {  // next batch: waits for its table load (once per 64 tiles)
        k0 = k;
        phys_vec = table_batch(k0);
      }
      int32_t phys = __builtin_amdgcn_readlane(phys_vec, k - k0);
      phys = phys < 0 ? 0 : (phys >= p.num_pages ? p.num_pages - 1 : phys);
      const char* tile = p.k + ((int64_t)phys * page_b + (int64_t)(16 * c.u) * ts_b + head_off_b);
      const int nvalid = cursor_valid(c);
#pragma unroll
      for (int u = 0; u < IPW; ++u) {
        const int64_t off = src_slot0[u] + ((nvalid == 16 || src_key[u] < nvalid) ? src_key_off[u] : 0);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(tile + off),
                                         (__attribute__((address_space(3))) void*)(ring + 1024 * (wave * IPW + u)),
                                         16, 0, 2 /* nt */);
      }
    } else {
      // sub-tiles 2k and 2k+1 (the batch is refilled at even sub-tiles, so both
      // are in it)
      const int ks = 2 * k;
      if (ks - k0 >= 64) {
        k0 = ks;
        sub_batch(k0, table_batch(k0));
      }
      const char* tile[2];
      int nv[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)poff_vec, ks + h - k0);
        const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)((uint64_t)poff_vec >> 32), ks + h - k0);
        tile[h] = p.k + ((int64_t)(((uint64_t)hi << 32) | lo) + head_off_b);
        nv[h] = __builtin_amdgcn_readlane(nv_vec, ks + h - k0);
      }
      // a second sub-tile past the end re-reads the first one's slot 0: its
      // page is not the request's (a table pad may point anywhere)
      if (nv[1] <= 0) tile[1] = tile[0];
#pragma unroll
      for (int u = 0; u < IPW; ++u) {
        const int h = src_half[u];
        const int nvalid = h == 0 ? nv[0] : nv[1];
        const int64_t off = src_slot0[u] + ((nvalid == 16 || src_key[u] < nvalid) ? src_key_off[u] : 0);
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>((h == 0 ? tile[0] : tile[1]) + off),
                                         (__attribute__((address_space(3))) void*)(ring + 1024 * (wave * IPW + u)),
                                         16, 0, 2 /* nt */);
      }
    }
  };

  // MFMA operands of a staged tile (LDS addresses are lane constants).
  //  16-bit K/V: V^T comes straight from transposing LDS reads
  //  (ds_read_b64_tr_b16), PV MFMA j covering head dims 16j .. 16j+15 (the
  //  blocked output layout).  Within each 16-lane group, lane r of such a read
  //  receives element r%4 of the 8-byte pieces addressed by lanes
  //  r/4 + 4e, e = 0..3 of its group.  So the lane with a = l%4,
  //  e = (l%16)/4 addresses dims 16j + 4a .. +3 of key 4*(l/16) + e, and lane
  //  l receives dim 16j + l%16 of keys 4*(l/16) + e: the A operand of V^T.
  //  fp8 K/V: 8-bit transposing reads (ds_read_b64_tr_b8), then an exact
  //  fp8 -> 16-bit decode; same blocked layout.  Within each 16-lane group,
  //  lane 8a+b of such a read receives byte b of the 8-byte pieces addressed
  //  by lanes 2e+a, e = 0..7 of its group.  Read p serves PV MFMAs 2p and
  //  2p+1: the lane with e = (l%16)/2, a = l%2 addresses key 4*(l/16) + e%4,
  //  head dims 16*(2p + e/4) + 8a .. +7, so lane l receives dim 16*(2p) + l%16
  //  of keys 4*(l/16) + 0..3 in bytes 0..3 and dim 16*(2p+1) + l%16 of the
  //  same keys in bytes 4..7.
  constexpr bool TR = KV != K_FP8;
  constexpr int NVL = TR ? VPL : VPL / 2;
  int k_lds[G::KLD], v_lds[NVL];
#pragma unroll
  for (int i = 0; i < G::KLD; ++i) {
    const int t = c16, c = 4 * i + g4;
    k_lds[i] = 16 * G::chunk_pos(t, c);
  }
  if constexpr (TR) {
    const int t = 4 * g4 + (c16 >> 2), a = c16 & 3;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int cv = G::CPK / 2 + 2 * j + (a >> 1);  // 32 bytes of V per j, 8 per a
      v_lds[j] = 16 * G::chunk_pos(t, cv) + 8 * (a & 1);
    }
  } else {
    const int e = c16 >> 1, a = c16 & 1;
    const int t = 4 * g4 + (e & 3);
#pragma unroll
    for (int pp = 0; pp < VPL / 2; ++pp) {
      const int cv = G::CPK / 2 + 2 * pp + (e >> 2);  // 16 bytes of V per PV MFMA
      v_lds[pp] = 16 * G::chunk_pos(t, cv) + 8 * a;
    }
  }
  auto read_k = [&](auto sc, Frags<D, QT>& f, int hoff = 0) {
    const char* st = stage_buf(sc) + hoff;
    if constexpr (TR) {
#pragma unroll
      for (int kc = 0; kc < G::NKC; ++kc) f.kf[kc] = *reinterpret_cast<const u32x4*>(st + k_lds[kc]);
    } else {
      u32x4 rk[G::KLD];
#pragma unroll
      for (int i = 0; i < G::KLD; ++i) rk[i] = *reinterpret_cast<const u32x4*>(st + k_lds[i]);
      k_operands<D, KV, QT>(rk, f);
    }
  };
  auto read_v = [&](auto sc, Frags<D, QT>& f, int hoff = 0) {
    const char* st = stage_buf(sc) + hoff;
    if constexpr (TR) {
#pragma unroll
      for (int j = 0; j < VPL; ++j)
        f.vA[j] = bitcast<u32x2>(__builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(st + v_lds[j])));
    } else {
      constexpr int PV = QTypes<QT>::PV;
#pragma unroll
      for (int pp = 0; pp < VPL / 2; ++pp) {
        const auto x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) v2i32*)(st + v_lds[pp]));
        uint32_t lo, hi;
        fp8x4_to_16<PV>((uint32_t)x[0], lo, hi);
        f.vA[2 * pp] = u32x2{lo, hi};
        fp8x4_to_16<PV>((uint32_t)x[1], lo, hi);
        f.vA[2 * pp + 1] = u32x2{lo, hi};
      }
    }
  };
  f32x4 acc[VPL];
  float m_run = kNegInf, l_run = 0.f;
#pragma unroll
  for (int j = 0; j < VPL; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // causal bounds of this lane's row; tiles inside [lo_max, hi_min] need no mask
  int row_hi = 0, row_lo = 0, hi_min = 0, lo_max = 0;
  if constexpr (CAUSAL) {
    const int Lr = pr.sv.len;
    row_hi = Lr - p.sq + (row0 + c16) / p.G;
    row_lo = p.window_left >= 0 ? row_hi - p.window_left : INT32_MIN;
    hi_min = Lr - p.sq;
    lo_max = p.window_left >= 0 ? Lr - 1 - p.window_left : INT32_MIN;
  }

  Cursor ci = cursor_at0();  // next tile to issue
  Cursor cc = cursor_at0();  // next tile to consume
  // prologue: tiles 0 .. NBUF-2 into stages 0 .. NBUF-2
  auto prologue = [&](auto sc) {
    constexpr int s = decltype(sc)::value;
    if constexpr (s < NBUF - 1) {
      if (s < n_tiles) {
        issue_tile(s, ci, sc);
        if constexpr (KT == 16) advance(ci);
      }
    }
  };
  static_all<0, NBUF - 1>([&](auto sc) {
    prologue(sc);
    return true;
  });
  // Settle the query fragments (and the first table batch) here, behind the
  // prologue's loads.  Left to the first use inside the tile loop, the wait
  // would stay in the loop and, merged with the ring loads of the previous
  // iteration, drain every load in flight on each tile.
#pragma unroll
  for (int i = 0; i < D / 32; ++i) asm volatile("" ::"v"(qf[i]));
  asm volatile("" ::"v"(phys_vec));

  // Tile k sits in stage k % NBUF; returns false once every tile is done.
  auto step = [&](auto sc, int k) -> bool {
    constexpr int s = decltype(sc)::value;
    if (k >= n_tiles) return false;
    // tiles issued after k by this wave: min(NBUF-2, n_tiles-1-k); wait for the rest
    wait_tiles_ahead<IPW, NBUF - 2>(min(NBUF - 2, n_tiles - 1 - k));
    // Every wave's part of tile k has landed and every wave has consumed tile
    // k-1 (its stage is refilled next).  A bare s_barrier: the usual
    // workgroup fence would also wait for the tiles still in flight.
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    // Refill tile k-1's stage with tile k+NBUF-1, issued from inside tile k's
    // work right after its S^T MFMAs: a wave issuing ring loads can stall while
    // the memory system pushes back, and its MFMAs then run meanwhile (the
    // fp8-query block measured 2-3% faster than issuing right after the barrier).
    auto refill = [&]() {
      if (k + NBUF - 1 < n_tiles) {
        issue_tile(k + NBUF - 1, ci, std::integral_constant<int, (s + NBUF - 1) % NBUF>{});
        if constexpr (KT == 16) advance(ci);
      }
    };
    const int nvalid = cursor_valid(cc);
    const int key0 = cc.tok0;
    advance(cc);
    if constexpr (KT == 32) {
      const int nvalid1 = cursor_valid(cc);
      advance(cc);
      Frags<D, QT> f0, f1;
      read_k(sc, f0);
      read_k(sc, f1, G::TILE_BYTES);
      // V^T stays fp8 in registers until each P.V MFMA converts its own part
      v2i32 rv[2][VPL / 2];
      auto vload = [&]() {
        const char* st = stage_buf(sc);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int pp = 0; pp < VPL / 2; ++pp)
            rv[h][pp] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) v2i32*)(st + h * G::TILE_BYTES + v_lds[pp]));
      };
      auto vop = [&](int j) -> u32x4 {
        constexpr int PV = QTypes<QT>::PV;
        uint32_t a0, a1, b0, b1;
        fp8x4_to_16<PV>((uint32_t)rv[0][j >> 1][j & 1], a0, a1);
        fp8x4_to_16<PV>((uint32_t)rv[1][j >> 1][j & 1], b0, b1);
        return u32x4{a0, a1, b0, b1};
      };
      attend_tile32<D, QT>(f0, f1, qf, acc, m_run, l_run, p.qk_scale_log2, nvalid, nvalid1, g4, refill,
                           vload, vop);
      return true;
    }
    Frags<D, QT> f;
    const bool on = CAUSAL && (key0 + 15 > hi_min || key0 < lo_max);
    // V^T is read only after the softmax, so it is not live across it: 96
    // instead of 108 VGPRs for the bf16 block, five waves per SIMD
    read_k(sc, f);
    attend_tile<D, QT, CAUSAL>(f, qf, acc, m_run, l_run, p.qk_scale_log2, 0.f, nvalid, g4, key0,
                               RowMask{on, row_hi, row_lo}, refill, [&]() { read_v(sc, f); });
    return true;
  };
  for (int k = 0;; k += NBUF)
    if (!static_all<0, NBUF>([&](auto sc) { return step(sc, k + decltype(sc)::value); })) break;

  l_run = sum_across_groups(l_run);
  float* lse_base = p.lse;
  void* o_base = p.out;
  if (p.partial) {
    lse_base = p.lse + (int64_t)split * p.split_stride_lse;
    o_base = reinterpret_cast<float*>(p.out) + (int64_t)split * p.split_stride_o;
  }
  // The lane index is derived afresh here (v_mbcnt) instead of kept from the
  // start, so no row-index value stays live across the tile loop: that frees
  // the VGPR the dense bf16 kernel needs for five waves per SIMD.
  int lane_now;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(lane_now));
  const int rr = row0 + (lane_now & 15);
  if (rr < p.R) {
    int G = p.G;  // opaque copy: no reciprocal of G kept from before the loop
    asm volatile("" : "+s"(G));
    const int t = rr / G, gg = rr % G;
    const int64_t orow = ((int64_t)item * p.sq + t) * p.Hq + kvh * p.G + gg;
    store_tile<D, true>(acc, m_run, l_run, p.v_scale, o_base, p.out_kind, lse_base, orow, p.partial,
                        lane_now >> 4);
  }
}

// ================================================================================
// dash_shared_kernel: DASH attention (dash_attention page, flash_dash_attention:
// one query against the valid rows of its gathered segments) with the K and V
// rows of HP kv heads staged through a two-stage LDS ring.
//   work item:  (query, group of HP consecutive kv heads); the group's part of
//               a token row (HP*D contiguous elements of K, the same of V) is
//               fetched by direct-to-LDS loads of 16-byte chunks.
//   waves:      HP, wave w serving kv head w of the group (its G query heads
//               are the rows of one 16-row tile).
//   fused (PARTS = false): the query's live keys are numbered across its
//               segments, 16 per tile (as the fused mode of attn_kernel), each
//               segment's bias is added to its logits and one online softmax
//               runs over all of them.
//   partials (PARTS = true): each segment is cut into its own tiles and gets
//               its own softmax; when its last tile is done the wave writes the
//               segment's normalised output and LSE (fp32) for the combine.
//   Slots past a tile's last live key fetch its first key and are masked.
// Each staged head uses attn_shared_kernel's tile layout (Geo::chunk_pos).
// Tile k sits in stage k % 2.  A wave reads all of its K and V operands as
// soon as the tile has landed; once every wave has, the stage takes tile k+2,
// so two tiles are in flight while a wave computes or waits.
// ================================================================================
template <int D, int KV, int HP, bool PARTS>
__global__ __launch_bounds__(HP * 64) void dash_shared_kernel(const AttnParams p) {
  using G = Geo<D, KV>;
  constexpr int KB = G::KB;
  constexpr int VPL = G::VPL;
  constexpr int SUB = G::TILE_BYTES;     // one kv head's staged tile
  constexpr int IPW = G::IPT;            // direct-to-LDS loads per wave per tile
  static_assert(KV != K_FP8, "16-bit K/V only");
  static_assert(SUB % 1024 == 0, "each 1 KiB load stays inside one head's staged tile");
  constexpr int QT = KV;
  __shared__ __attribute__((aligned(1024))) char ring0[HP * SUB];
  __shared__ __attribute__((aligned(1024))) char ring1[HP * SUB];
  auto stage_buf = [&](auto sc) -> char* {
    if constexpr (decltype(sc)::value == 0) return ring0;
    else return ring1;
  };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int g4 = lane >> 4;
  const int c16 = lane & 15;

  const int groups = p.Hkv / HP;
  const int n = (int)(blockIdx.x / (uint32_t)groups);
  const int grp = (int)(blockIdx.x % (uint32_t)groups);
  const int kvh = grp * HP + wave;

  const SegLanes sl = seg_lanes(p, n, lane);
  int n_tiles = (sl.n_keys + 15) >> 4;
  // partials: lane g also holds segment g's first tile and its tile count
  int seg_t0 = 0x7fffffff, seg_t1 = 0x7fffffff;  // tiles [seg_t0, seg_t1)
  if constexpr (PARTS) {
    const int nt = lane <= p.topk ? (sl.cum_end - sl.cum_start + 15) >> 4 : 0;
    int cum = nt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(cum, off, 64);
      if (lane >= off) cum += o;
    }
    n_tiles = __builtin_amdgcn_readlane(cum, 63);
    if (lane <= p.topk) {
      seg_t1 = cum;
      seg_t0 = cum - nt;
    }
  }
  const int64_t ts_b = p.token_stride * KB;
  // the group's part of the query's first row, in K (V adds the V - K distance)
  const int64_t qoff_b = (int64_t)n * (p.topk * p.bs + p.local) * ts_b +
                         (int64_t)grp * HP * p.head_stride * KB;

  typename QTypes<QT>::QOp qf[D / 32];
  load_q<D, KV, QT>(qf, p.q, 0, p.R, p.G, kvh, n, 1, p.Hq, g4, c16);

  // Lane constants of this wave's loads: load u writes LDS chunk position
  // 64*(wave*IPW + u) + lane of the stage, which holds chunk c of key slot t
  // of the wave's own head (heads one after another, each in
  // attn_shared_kernel's layout).
  const int64_t vk = p.v - p.k;
  int64_t src_c[IPW];
  int src_t[IPW];
#pragma unroll
  for (int u = 0; u < IPW; ++u) {
    const int q = 64 * u + lane;
    const int t = q / G::CPK;
    const int c = (q % G::CPK) ^ G::swz(t, q % G::CPK);
    src_c[u] = (c < G::CPK / 2 ? 16 * c : vk + 16 * (c - G::CPK / 2)) +
               (int64_t)wave * p.head_stride * KB;
    src_t[u] = t;
  }
  const uint32_t tsb = (uint32_t)ts_b;  // 16 * tsb < 2^31 (checked at the boundary)

  // partials: segment of tile k, the tile's first row within the query and
  // its live keys
  auto part_tile = [&](int k, int& g, int& row0, int& nvalid) {
    g = __builtin_amdgcn_readfirstlane(__builtin_popcountll(__ballot(seg_t1 <= k)));
    const int j = k - __builtin_amdgcn_readlane(seg_t0, g);
    row0 = __builtin_amdgcn_readlane(sl.adj + sl.cum_start, g) + 16 * j;
    nvalid = min(16, __builtin_amdgcn_readlane(sl.cum_end - sl.cum_start, g) - 16 * j);
  };
  auto issue_tile = [&](int k, auto sc) {
    int key0, nvalid, d[IPW], row[IPW];
    if constexpr (PARTS) {
      int g, row0;
      part_tile(k, g, row0, nvalid);
      key0 = 0;
#pragma unroll
      for (int u = 0; u < IPW; ++u) {
        d[u] = src_t[u] < nvalid ? src_t[u] : 0;
        row[u] = row0;
      }
    } else {
      key0 = 16 * k;
      const int g0 = seg_of_key(sl, key0);
      nvalid = min(16, sl.n_keys - key0);
#pragma unroll
      for (int u = 0; u < IPW; ++u) d[u] = src_t[u] < nvalid ? src_t[u] : 0;
      seg_field(sl, p.topk, key0, g0, d, sl.adj, row);
    }
    const char* base = p.k + uniform64(qoff_b);
    char* st = stage_buf(sc) + wave * SUB;
#pragma unroll
    for (int u = 0; u < IPW; ++u) {
      const uint64_t off = (uint64_t)(uint32_t)(row[u] + key0 + d[u]) * tsb;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(base + (off + src_c[u])),
                                       (__attribute__((address_space(3))) void*)(st + 1024 * u),
                                       16, 0, 2 /* nt */);
    }
  };

  // MFMA operands of the wave's head in a stage (as in attn_shared_kernel)
  int k_lds[G::KLD], v_lds[VPL];
#pragma unroll
  for (int i = 0; i < G::KLD; ++i) k_lds[i] = wave * SUB + 16 * G::chunk_pos(c16, 4 * i + g4);
  {
    const int t = 4 * g4 + (c16 >> 2), a = c16 & 3;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int cv = G::CPK / 2 + 2 * j + (a >> 1);
      v_lds[j] = wave * SUB + 16 * G::chunk_pos(t, cv) + 8 * (a & 1);
    }
  }

  f32x4 acc[VPL];
  float m_run = kNegInf, l_run = 0.f;
#pragma unroll
  for (int j = 0; j < VPL; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (0 < n_tiles) issue_tile(0, std::integral_constant<int, 0>{});
  if (1 < n_tiles) issue_tile(1, std::integral_constant<int, 1>{});
  // Settle the query fragments here, outside the tile loop.  This waits for
  // the two tiles just issued as well; with them still pending at the loop
  // entry, the compiler's tracking of direct-to-LDS writes loses the stages
  // apart and drains every load in flight before each read of stage 0.
#pragma unroll
  for (int i = 0; i < D / 32; ++i) asm volatile("" ::"v"(qf[i]));

  auto step = [&](auto sc, int k) -> bool {
    if (k >= n_tiles) return false;
    wait_tiles_ahead<IPW, 1>(min(1, n_tiles - 1 - k));
    // every wave's part of tile k has landed (bare s_barrier: a workgroup
    // fence would also wait for the tile still in flight)
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const char* st = stage_buf(sc);
    Frags<D, QT> f;
#pragma unroll
    for (int kc = 0; kc < G::NKC; ++kc) f.kf[kc] = *reinterpret_cast<const u32x4*>(st + k_lds[kc]);
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      f.vA[j] = bitcast<u32x2>(__builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(st + v_lds[j])));
    int key0 = 16 * k, nvalid, g = 0, row0 = 0;
    f32x4 kbias = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (PARTS) {
      part_tile(k, g, row0, nvalid);
      if (k == __builtin_amdgcn_readlane(seg_t0, g)) {  // a segment starts: fresh softmax
        m_run = kNegInf;
        l_run = 0.f;
#pragma unroll
        for (int j = 0; j < VPL; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    } else {
      nvalid = min(16, sl.n_keys - key0);
      // bias of the segment of each of the lane's keys 4*g4 + i (the S^T layout)
      int d[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) d[i] = 4 * g4 + i;
      seg_field(sl, p.topk, key0, seg_of_key(sl, key0), d, __float_as_int(sl.bias), b);
#pragma unroll
      for (int i = 0; i < 4; ++i) kbias[i] = __int_as_float(b[i]);
    }
    // once every wave's reads of the stage have returned, it takes tile k+2;
    // issued behind the S^T MFMAs, which run while the loads go out
    auto refill = [&]() {
      __builtin_amdgcn_s_waitcnt(kLgkmcnt0);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_barrier();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      if (k + 2 < n_tiles) issue_tile(k + 2, sc);
    };
    attend_tile<D, QT, false, !PARTS, !PARTS>(f, qf, acc, m_run, l_run, p.qk_scale_log2, 0.f,
                                              nvalid, g4, key0, RowMask{false, 0, 0}, refill,
                                              NoHook{}, kbias);
    if constexpr (PARTS) {
      if (k + 1 == __builtin_amdgcn_readlane(seg_t1, g)) {  // the segment's last tile
        const float l_tot = sum_across_groups(l_run);
        if (c16 < p.R)
          store_tile<D, true>(acc, m_run, l_tot, p.v_scale, p.out, p.out_kind, p.lse,
                              ((int64_t)n * (p.topk + 1) + g) * p.Hq + kvh * p.G + c16, true, g4);
      }
    }
    return true;
  };
  for (int k = 0;; k += 2) {
    if (!step(std::integral_constant<int, 0>{}, k)) break;
    if (!step(std::integral_constant<int, 1>{}, k + 1)) break;
  }

  if constexpr (!PARTS) {
    l_run = sum_across_groups(l_run);
    if (c16 < p.R)
      store_tile<D, true>(acc, m_run, l_run, p.v_scale, p.out, p.out_kind, p.lse,
                          (int64_t)n * p.Hq + kvh * p.G + c16, false, g4);
  }
}

// ---- instantiation table ------------------------------------------------------------
namespace {

// LDS ring depth of attn_shared_kernel.  Three 8 KiB stages let five bf16
// workgroups share a CU's 160 KiB of LDS (four stages allow only four), and
// with V read late the kernel fits five waves per SIMD: more waves issuing
// loads at once (C3 420 -> 407 us, fp8-query block 291 -> 277 us).  Deeper
// rings measured no faster at equal occupancy (3 ~ 4 ~ 5 > 6 > 8).
constexpr int kRingStages = 3;

using KernelFn = void (*)(AttnParams);

template <int D, int KV, int QT, int MODE, bool C>
KernelFn pick_keys(int RT, int NW) {
  if (RT == 1 && NW == 4) return attn_kernel<D, 1, 4, KV, QT, MODE, C>;
  if (RT == 1 && NW == 2) return attn_kernel<D, 1, 2, KV, QT, MODE, C>;
  if (RT == 1 && NW == 1) return attn_kernel<D, 1, 1, KV, QT, MODE, C>;
  if (RT == 2 && NW == 2) return attn_kernel<D, 2, 2, KV, QT, MODE, C>;
  if (RT == 4 && NW == 1) return attn_kernel<D, 4, 1, KV, QT, MODE, C>;
  return nullptr;
}

template <int D, int KV, int QT, bool C>
KernelFn pick_rows(int NW) {
  constexpr int IPT = Geo<D, KV>::IPT;
  constexpr int KT = (QT == K_FP8 && !C) ? 32 : 16;
  constexpr int IPT2 = IPT * KT / 16;
  if constexpr (IPT2 % 8 == 0)
    if (NW == 8) return attn_shared_kernel<D, 8, KV, QT, kRingStages, C, KT>;
  if constexpr (IPT2 % 4 == 0)
    if (NW == 4) return attn_shared_kernel<D, 4, KV, QT, kRingStages, C, KT>;
  if (NW == 2) return attn_shared_kernel<D, 2, KV, QT, kRingStages, C, KT>;
  return nullptr;
}

template <int D, int KV, int QT, int MODE>
KernelFn pick_kind(const LaunchShape& s) {
  if constexpr (MODE == MODE_PAGED) {
    if (s.rows_split)
      return s.causal ? pick_rows<D, KV, QT, true>(s.NW) : pick_rows<D, KV, QT, false>(s.NW);
    return s.causal ? pick_keys<D, KV, QT, MODE, true>(s.RT, s.NW)
                    : pick_keys<D, KV, QT, MODE, false>(s.RT, s.NW);
  } else {
    if (s.rows_split || s.causal) return nullptr;
    return pick_keys<D, KV, QT, MODE, false>(s.RT, s.NW);
  }
}

template <int D, int MODE>
KernelFn pick_types(const LaunchShape& s) {
  if (s.kv_kind == K_BF16 && s.q_kind == K_BF16) return pick_kind<D, K_BF16, K_BF16, MODE>(s);
  if (s.kv_kind == K_FP16 && s.q_kind == K_FP16) return pick_kind<D, K_FP16, K_FP16, MODE>(s);
  if constexpr (MODE == MODE_PAGED) {
    if (s.kv_kind == K_FP8 && s.q_kind == K_BF16) return pick_kind<D, K_FP8, K_BF16, MODE>(s);
    if (s.kv_kind == K_FP8 && s.q_kind == K_FP16) return pick_kind<D, K_FP8, K_FP16, MODE>(s);
    if (s.kv_kind == K_FP8 && s.q_kind == K_FP8) return pick_kind<D, K_FP8, K_FP8, MODE>(s);
  }
  return nullptr;
}

template <int MODE>
KernelFn pick_d(const LaunchShape& s) {
  if (s.D == 128) return pick_types<128, MODE>(s);
  if (s.D == 64) return pick_types<64, MODE>(s);
  return nullptr;
}

KernelFn pick(const LaunchShape& s) {
  switch (s.mode) {
    case MODE_PAGED: return pick_d<MODE_PAGED>(s);
    case MODE_SEGMENT: return pick_d<MODE_SEGMENT>(s);
    case MODE_SEGMENT_FUSED: return pick_d<MODE_SEGMENT_FUSED>(s);
    default: return nullptr;
  }
}

}  // namespace

bool attention_supported(const LaunchShape& s) { return pick(s) != nullptr; }

int shared_tile_loads(int D, int kv_kind) {
  const int kb = kv_kind == K_FP8 ? 1 : 2;
  return 16 * 2 * D * kb / 1024;
}

namespace {
template <bool PARTS>
KernelFn pick_dash_mode(int D, int kv_kind) {
  if (D == 128 && kv_kind == K_BF16) return dash_shared_kernel<128, K_BF16, kDashHeads, PARTS>;
  if (D == 128 && kv_kind == K_FP16) return dash_shared_kernel<128, K_FP16, kDashHeads, PARTS>;
  if (D == 64 && kv_kind == K_BF16) return dash_shared_kernel<64, K_BF16, kDashHeads, PARTS>;
  if (D == 64 && kv_kind == K_FP16) return dash_shared_kernel<64, K_FP16, kDashHeads, PARTS>;
  return nullptr;
}
KernelFn pick_dash(int D, int kv_kind, bool parts) {
  return parts ? pick_dash_mode<true>(D, kv_kind) : pick_dash_mode<false>(D, kv_kind);
}
}  // namespace

bool dash_shared_supported(int D, int kv_kind, int G, int Hkv) {
  return pick_dash(D, kv_kind, false) != nullptr && G >= 1 && G <= 16 && Hkv % kDashHeads == 0;
}

hipError_t launch_dash_shared(const AttnParams& p, int D, int kv_kind, hipStream_t stream) {
  KernelFn fn = pick_dash(D, kv_kind, p.partial != 0);
  if (!fn || p.G > 16 || p.R != p.G || p.Hkv % kDashHeads) return hipErrorInvalidValue;
  const int64_t grid = (int64_t)p.items * (p.Hkv / kDashHeads);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(64 * kDashHeads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnParams& p, const LaunchShape& s, int64_t grid,
                            hipStream_t stream) {
  KernelFn fn = pick(s);
  if (!fn) return hipErrorInvalidValue;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const size_t lds = s.rows_split ? 0 : merge_lds_bytes(s.D, s.NW, p.R, s.RT);
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(64 * s.NW), lds, stream, p);
  return hipGetLastError();
}

}  // namespace pa
