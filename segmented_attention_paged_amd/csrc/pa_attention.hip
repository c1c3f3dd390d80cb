// Paged / segmented attention kernel for gfx950 (CDNA4, wave64, MFMA).
//
// One workgroup = NW waves = one work item:
//   paged:          (request, kv head, row group, split)
//   segment:        (query, segment, kv head, row group)
//   segment fused:  (query, kv head, row group)
// The rows of a work item are the G query heads of one kv head times the
// query block (row r -> token r / G, head kvh*G + r % G), packed into 16-row
// MFMA tiles (RT tiles per wave).  Keys are consumed in tiles of 16 slots of
// one page.  Waves of a workgroup take tiles round-robin, each keeping its
// own online-softmax state; the states are merged through LDS at the end.
//
// Per 16-key tile and 16-row tile:
//   S^T = K Q^T   D/32  x v_mfma_f32_16x16x32_{bf16,f16}; K is the A operand,
//                 loaded straight from the page: lane l reads 16 contiguous
//                 bytes of key l%16 (no LDS, no shuffles).
//   online softmax in fp32 registers (log2 domain, v_exp_f32).
//   O^T += V^T P^T  D/16 x v_mfma_f32_16x16x16_{bf16,f16}; P^T is the S^T
//                 accumulator re-packed to 16 bits in place (same lane layout),
//                 V^T is built from 4 keys x 16 bytes per lane with byte
//                 permutes: A-row m of MFMA j is head-dim VPL*m + j.
// fp8 (e4m3fn) K/V are decoded exactly to the query's 16-bit type with the
// gfx950 pk conversions; k_scale folds into the logit scale and v_scale into
// the epilogue (vllm.v1.attention.backends.flashinfer_ts, forward:
// bmm1_scale / bmm2_scale).

#include "pa_device.h"
#include "pa_kernels.h"
#include "pa_plan.h"

namespace pa {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();

struct TileInfo {
  const char* kp;  // byte address of slot 0 of the tile, head kvh, in K
  const char* vp;  // same in V
  int nvalid;      // slots [0, nvalid) hold visible keys (1..16)
  float bias;      // log2-domain logit bias of the tile (fused segments)
};

template <int VDW>
__device__ __forceinline__ void load_v(uint32_t (&dst)[VDW], const char* src) {
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

}  // namespace

template <int D, int RT, int NW, int KV, int QT, int MODE>
__global__ __launch_bounds__(NW * 64) void attn_kernel(const AttnParams p) {
  static_assert(D == 64 || D == 128, "head_dim");
  constexpr int KB = (KV == K_FP8) ? 1 : 2;  // bytes per stored K/V element
  constexpr int NKC = D / 32;                // QK MFMAs per row tile
  constexpr int VPL = D / 16;                // PV MFMAs per row tile = head-dim values per lane per key
  constexpr int KLD = D * KB / 64;           // 16-byte K loads per lane per tile
  constexpr int VDW = VPL * KB / 4;          // V dwords per lane per key
  constexpr int ROWS = RT * 16;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g4 = lane >> 4;
  const int c16 = lane & 15;

  // ---- work item ------------------------------------------------------------
  int64_t bid = blockIdx.x;
  int split = 0;
  if constexpr (MODE == MODE_PAGED) {
    split = (int)(bid % p.S);
    bid /= p.S;
  }
  const int rg = (int)(bid % p.RG);
  bid /= p.RG;
  const int kvh = (int)(bid % p.Hkv);
  const int item = (int)(bid / p.Hkv);

  const int64_t ts_b = p.token_stride * KB;
  const int64_t head_off_b = (int64_t)kvh * p.head_stride * KB;

  int n_tiles = 0;
  int qb = item;  // request index used to address q and the output rows
  // paged
  SeqView sv{};
  SplitRange sr{};
  int TPP = 1, tok_end = 0;
  // segment
  int64_t seg_tok0 = 0;
  int seg_used = 0;
  // fused segments: lane g holds the description of segment g
  int f_used = 0, f_tiles = 0, f_cum_end = 0x7fffffff;
  int64_t f_base = 0;
  float f_bias = 0.f;

  if constexpr (MODE == MODE_PAGED) {
    sv = seq_view(p.seq_lens[item], p.window, p.sq, p.P, p.bt_width);
    sr = split_range(sv, p.P, p.S, p.chunk, split);
    TPP = (p.P + 15) >> 4;
    tok_end = sr.tok0 + sr.n_tok;
    if (sr.n_pages > 0) {
      const int last_count = sr.n_tok - (sr.n_pages - 1) * p.P;
      n_tiles = (sr.n_pages - 1) * TPP + ((last_count + 15) >> 4);
    }
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
    const int Gs = p.topk + 1;
    const int n = item;
    if (lane < Gs) {
      const int cap = lane < p.topk ? p.bs : p.local;
      int u = p.used[(int64_t)n * Gs + lane];
      u = u < 0 ? 0 : (u > cap ? cap : u);
      f_used = u;
      f_tiles = (u + 15) >> 4;
      f_base = (int64_t)n * (p.topk * p.bs + p.local) + (lane < p.topk ? lane * p.bs : p.topk * p.bs);
      f_bias = lane < p.topk ? p.bias[(int64_t)n * p.topk + lane] * kLog2e : 0.f;
    }
    // inclusive prefix sum of tile counts across lanes
    int cum = f_tiles;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(cum, off, 64);
      if (lane >= off) cum += o;
    }
    n_tiles = __shfl(cum, 63, 64);
    f_cum_end = lane < Gs ? cum : 0x7fffffff;
    qb = n;
  }

  // ---- query fragments (B operand of S^T = K Q^T) -----------------------------
  u32x4 qf[RT][NKC];
  const int row_base = rg * ROWS;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int rr = row_base + rt * 16 + c16;
    if (rr < p.R) {
      const int t = rr / p.G, gg = rr % p.G;
      const int h = kvh * p.G + gg;
      const uint16_t* qrow =
          reinterpret_cast<const uint16_t*>(p.q) + (((int64_t)qb * p.sq + t) * p.Hq + h) * D;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const int d = (KV == K_FP8) ? 64 * (kc >> 1) + 16 * g4 + 8 * (kc & 1) : 32 * kc + 8 * g4;
        qf[rt][kc] = *reinterpret_cast<const u32x4*>(qrow + d);
      }
    } else {
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) qf[rt][kc] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  // ---- per-wave page index cache (paged): lane i holds the pool page of the
  // wave's tile k0 + i ---------------------------------------------------------
  int32_t phys_vec = 0;
  int k0 = -64;
  const int32_t* trow = nullptr;
  if constexpr (MODE == MODE_PAGED) trow = p.block_table + (int64_t)item * p.bt_stride;

  auto tile_info = [&](int k) -> TileInfo {
    const int it = wave + NW * k;
    TileInfo ti;
    ti.bias = 0.f;
    if constexpr (MODE == MODE_PAGED) {
      if (k - k0 >= 64) {
        k0 = k;
        const int itl = wave + NW * (k0 + lane);
        int32_t ph = 0;
        if (itl < n_tiles) {
          const int page = sr.first_page + itl / TPP;
          ph = trow[table_column(sv, page, p.bt_width)];
          ph = ph < 0 ? 0 : (ph >= p.num_pages ? p.num_pages - 1 : ph);
        }
        phys_vec = ph;
      }
      const int32_t phys = __builtin_amdgcn_readlane(phys_vec, k - k0);
      const int pin = it / TPP, u = it - pin * TPP;
      const int page = sr.first_page + pin;
      const int slot0 = 16 * u;
      const int tok0 = page * p.P + slot0;
      int nv = p.P - slot0;
      if (nv > 16) nv = 16;
      if (tok_end - tok0 < nv) nv = tok_end - tok0;
      ti.nvalid = nv;
      const int64_t off = ((int64_t)phys * p.page_stride + (int64_t)slot0 * p.token_stride) * KB + head_off_b;
      ti.kp = p.k + off;
      ti.vp = p.v + off;
    } else if constexpr (MODE == MODE_SEGMENT) {
      const int64_t tok = seg_tok0 + 16 * it;
      int nv = seg_used - 16 * it;
      ti.nvalid = nv > 16 ? 16 : nv;
      const int64_t off = tok * ts_b + head_off_b;
      ti.kp = p.k + off;
      ti.vp = p.v + off;
    } else {
      // segment holding tile `it`: number of segments that end at or before it
      const int gsel = __builtin_popcountll(__ballot(f_cum_end <= it));
      const int cend = __shfl(f_cum_end, gsel, 64);
      const int ntl = __shfl(f_tiles, gsel, 64);
      const int ul = __shfl(f_used, gsel, 64);
      const int64_t base = __shfl(f_base, gsel, 64);
      ti.bias = __shfl(f_bias, gsel, 64);
      const int lt = it - (cend - ntl);
      int nv = ul - 16 * lt;
      ti.nvalid = nv > 16 ? 16 : nv;
      const int64_t off = (base + 16 * lt) * ts_b + head_off_b;
      ti.kp = p.k + off;
      ti.vp = p.v + off;
    }
    return ti;
  };

  struct Raw {
    u32x4 k[KLD];
    uint32_t v[4][VDW];
  };
  auto load_tile = [&](Raw& r, const TileInfo& ti) {
    const int ks = c16 < ti.nvalid ? c16 : 0;  // invalid slots read slot 0 (masked below)
    const char* kl = ti.kp + ks * ts_b + 16 * g4;
#pragma unroll
    for (int i = 0; i < KLD; ++i) r.k[i] = *reinterpret_cast<const u32x4*>(kl + 64 * i);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int vs = 4 * g4 + i;
      vs = vs < ti.nvalid ? vs : 0;
      load_v<VDW>(r.v[i], ti.vp + vs * ts_b + VPL * KB * c16);
    }
  };

  f32x4 acc[RT][VPL];
  float m_run[RT], l_run[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    m_run[rt] = kNegInf;
    l_run[rt] = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j) acc[rt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto compute_tile = [&](const Raw& r, const TileInfo& ti) {
    // K fragments in the query's 16-bit type
    u32x4 kf[NKC];
    if constexpr (KV == K_FP8) {
#pragma unroll
      for (int c2 = 0; c2 < KLD; ++c2) {
        uint32_t a0, a1, a2, a3, b0, b1, b2, b3;
        fp8x4_to_16<QT>(r.k[c2][0], a0, a1);
        fp8x4_to_16<QT>(r.k[c2][1], a2, a3);
        fp8x4_to_16<QT>(r.k[c2][2], b0, b1);
        fp8x4_to_16<QT>(r.k[c2][3], b2, b3);
        kf[2 * c2] = u32x4{a0, a1, a2, a3};
        kf[2 * c2 + 1] = u32x4{b0, b1, b2, b3};
      }
    } else {
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) kf[kc] = r.k[kc];
    }
    // V^T fragments: vA[j] holds head-dim VPL*c16 + j of keys 4*g4 + 0..3
    uint32_t v16[4][VPL / 2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (KV == K_FP8) {
#pragma unroll
        for (int w = 0; w < VDW; ++w) fp8x4_to_16<QT>(r.v[i][w], v16[i][2 * w], v16[i][2 * w + 1]);
      } else {
#pragma unroll
        for (int w = 0; w < VDW; ++w) v16[i][w] = r.v[i][w];
      }
    }
    u32x2 vA[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int w = j >> 1;
      if ((j & 1) == 0)
        vA[j] = u32x2{lo_lo(v16[0][w], v16[1][w]), lo_lo(v16[2][w], v16[3][w])};
      else
        vA[j] = u32x2{hi_hi(v16[0][w], v16[1][w]), hi_hi(v16[2][w], v16[3][w])};
    }
    const bool partial_tile = ti.nvalid < 16;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) sacc = mfma_16x16x32<QT>(kf[kc], qf[rt][kc], sacc);
      float s[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = sacc[i] * p.qk_scale_log2 + ti.bias;
      if (partial_tile) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (4 * g4 + i >= ti.nvalid) s[i] = kNegInf;
      }
      float tmax = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      tmax = max_across_groups(tmax);
      const float m_new = fmaxf(m_run[rt], tmax);
      const float alpha = fast_exp2(m_run[rt] - m_new);
      float pr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pr[i] = fast_exp2(s[i] - m_new);
      l_run[rt] = l_run[rt] * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
      m_run[rt] = m_new;
      const u32x2 pB = u32x2{pack2<QT>(pr[0], pr[1]), pack2<QT>(pr[2], pr[3])};
#pragma unroll
      for (int j = 0; j < VPL; ++j) {
        acc[rt][j] *= alpha;
        acc[rt][j] = mfma_16x16x16<QT>(vA[j], pB, acc[rt][j]);
      }
    }
  };

  // ---- main loop: prefetch tile k+1 while computing tile k --------------------
  if (wave < n_tiles) {
    TileInfo ti = tile_info(0);
    Raw cur;
    load_tile(cur, ti);
    for (int k = 0;; ++k) {
      const bool more = wave + NW * (k + 1) < n_tiles;
      TileInfo tn = ti;
      Raw nxt;
      if (more) {
        tn = tile_info(k + 1);
        load_tile(nxt, tn);
      }
      compute_tile(cur, ti);
      if (!more) break;
      cur = nxt;
      ti = tn;
    }
  }

#pragma unroll
  for (int rt = 0; rt < RT; ++rt) l_run[rt] = sum_across_groups(l_run[rt]);

  // ---- epilogue ----------------------------------------------------------------
  auto out_row = [&](int rr, int64_t& orow) {
    const int t = rr / p.G, gg = rr % p.G;
    const int h = kvh * p.G + gg;
    orow = ((int64_t)qb * p.sq + t) * p.Hq + h;
    if constexpr (MODE == MODE_SEGMENT) orow = (int64_t)item * p.Hq + h;
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
      if (rr >= p.R) continue;
      int64_t orow;
      out_row(rr, orow);
      const float l = l_run[rt];
      const bool live = l > 0.f;
      const float inv = live ? p.v_scale / l : 0.f;
      if (live || !p.partial) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float vals[VPL];
#pragma unroll
          for (int j = 0; j < VPL; ++j) vals[j] = acc[rt][j][i] * inv;
          store_row<VPL>(o_base, orow * D + VPL * (4 * g4 + i), p.out_kind, vals);
        }
      }
      if (g4 == 0 && lse_base) lse_base[orow] = live ? (m_run[rt] + log2f(l)) * kLn2 : kNegInf;
    }
  } else {
    __shared__ float red_o[NW][ROWS][D + 4];
    __shared__ float red_m[NW][ROWS];
    __shared__ float red_l[NW][ROWS];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int row = rt * 16 + c16;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < VPL; ++j) red_o[wave][row][VPL * (4 * g4 + i) + j] = acc[rt][j][i];
      if (g4 == 0) {
        red_m[wave][row] = m_run[rt];
        red_l[wave][row] = l_run[rt];
      }
    }
    __syncthreads();
    constexpr int QD = D / 4;
    for (int e = threadIdx.x; e < ROWS * QD; e += NW * 64) {
      const int row = e / QD;
      const int dq = (e - row * QD) * 4;
      const int rr = row_base + row;
      if (rr >= p.R) continue;
      int64_t orow;
      out_row(rr, orow);
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, red_m[w][row]);
      float o[4] = {0.f, 0.f, 0.f, 0.f};
      float tot = 0.f;
      if (M != kNegInf) {
        float wgt[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          wgt[w] = fast_exp2(red_m[w][row] - M);
          tot += wgt[w] * red_l[w][row];
        }
        const float inv = p.v_scale / tot;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const float c = wgt[w] * inv;
#pragma unroll
          for (int q = 0; q < 4; ++q) o[q] += c * red_o[w][row][dq + q];
        }
      }
      const bool live = tot > 0.f;
      if (live || !p.partial) store_row<4>(o_base, orow * D + dq, p.out_kind, o);
      if (dq == 0 && lse_base) lse_base[orow] = live ? (M + log2f(tot)) * kLn2 : kNegInf;
    }
  }
}

// ---- instantiation table ------------------------------------------------------
namespace {

using KernelFn = void (*)(AttnParams);

template <int D, int RT, int NW, int KV, int QT, int MODE>
constexpr KernelFn kfn() {
  return attn_kernel<D, RT, NW, KV, QT, MODE>;
}

template <int D, int KV, int QT, int MODE>
KernelFn pick_rt_nw(int RT, int NW) {
  if (RT == 1 && NW == 4) return kfn<D, 1, 4, KV, QT, MODE>();
  if (RT == 1 && NW == 1) return kfn<D, 1, 1, KV, QT, MODE>();
  if (RT == 2 && NW == 2) return kfn<D, 2, 2, KV, QT, MODE>();
  if (RT == 4 && NW == 1) return kfn<D, 4, 1, KV, QT, MODE>();
  return nullptr;
}

template <int D, int MODE>
KernelFn pick_types(int kv, int q, int RT, int NW) {
  if (kv == K_BF16 && q == K_BF16) return pick_rt_nw<D, K_BF16, K_BF16, MODE>(RT, NW);
  if (kv == K_FP16 && q == K_FP16) return pick_rt_nw<D, K_FP16, K_FP16, MODE>(RT, NW);
  if constexpr (MODE == MODE_PAGED) {
    if (kv == K_FP8 && q == K_BF16) return pick_rt_nw<D, K_FP8, K_BF16, MODE>(RT, NW);
    if (kv == K_FP8 && q == K_FP16) return pick_rt_nw<D, K_FP8, K_FP16, MODE>(RT, NW);
  }
  return nullptr;
}

template <int MODE>
KernelFn pick_d(const LaunchShape& s) {
  if (s.D == 128) return pick_types<128, MODE>(s.kv_kind, s.q_kind, s.RT, s.NW);
  if (s.D == 64) return pick_types<64, MODE>(s.kv_kind, s.q_kind, s.RT, s.NW);
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

hipError_t launch_attention(const AttnParams& p, const LaunchShape& s, int64_t grid,
                            hipStream_t stream) {
  KernelFn fn = pick(s);
  if (!fn) return hipErrorInvalidValue;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(64 * s.NW), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pa
