// bf16 MFMA forward of pair-biased 3D attention for gfx950, head_dim 8, 16, 32.
//
// The MegaFold pages (gist.science technical summary, Methodik section 1
// "EvoFlash-3D") describe the method: the logits of a row are produced tile by
// tile in on-chip memory and normalised with an online, numerically stable
// softmax (Milakov and Gimelshein, "Online normalizer calculation for
// softmax"), so the R*H*N*N logit tensor never reaches HBM; the pair bias is
// added to every row.
//
// Mapping to CDNA4:
//  * the work is split into items of 128 queries of two rows (r, r+1) of one
//    head; a persistent grid of two 4-wave workgroups per compute unit walks
//    through them.  A wave owns 32 queries of both rows, so each bias tile it
//    loads serves two rows.  Tiles are transposed, S^T = K Q^T (keys x
//    queries), so a lane holds one query and the softmax needs no cross-lane
//    work except one exchange with lane l ^ 32 at the end;
//  * the key blocks (64 keys) of a workgroup's items form one stream: K and V
//    of both rows are staged in LDS by direct global -> LDS copies in a ring of
//    four stages, issued two blocks ahead of their use, so the next item's first
//    blocks arrive while the current one ends.  At each block boundary the
//    outstanding copies and bias loads are retired (one wait and one workgroup
//    barrier) and the next block's are issued;
//  * the two rows of a wave are processed in a ping-pong over 32-key tiles: while
//    the vector ALU exponentiates row 0's tile t, the matrix cores compute row 1's
//    logits of tile t and row 1's P V product of tile t - 1; then the roles swap
//    (row 1's exponentials beside row 0's logits of tile t + 1 and P V of tile t).
//    The matrix work of each half-step does not depend on its vector work, so
//    the two overlap within one wave.  Row 1 finishes an item half a step after
//    row 0, so the rows switch to the next item's queries one half-step apart;
//  * the MFMA accumulator of S^T starts from sqrt(d) * bias, read as four coalesced
//    1 KB loads from a pre-pass's tiled copy about one block ahead; the key mask
//    enters as one more 16-deep MFMA step on exact split-bf16 operands (a masked
//    key's operand holds -inf itself, so its logit is exactly -inf); so neither
//    costs vector ALU work.  One FMA per logit applies log2(e)/sqrt(d) and
//    subtracts the reference point;
//  * the softmax keeps a lazily moved reference point: it starts at 0 and moves
//    only when some lane's running sum leaves [2^-64, 2^64] (or no live key was
//    seen yet); the normaliser l is the fp32 sum of the fp32 probabilities, and
//    P^T packed to bf16 is the B operand of O^T += V^T P^T, with V^T from
//    transposing LDS reads;
//  * an item's trailing key blocks whose keys are masked in both rows are not
//    visited;
//  * each XCD works through one contiguous range of items, so its L2 holds one
//    head's bias and the rows' K, V while its workgroups use them.

#include <algorithm>
#include <type_traits>

#include "dma_common.h"

namespace evo {
namespace {

using namespace mfma;
using namespace dma;
using pipe::kBlk;
using pipe::Tile;

constexpr int kPpQueries = 128;            // queries per workgroup (32 per wave)

template <int D>
struct FwdStage {
  char kv[4 * Tile<D>::BYTES];  // 64 keys of K row 0, V row 0, K row 1, V row 1
  char kaug[2 * kBlk * 16];     // key-side split operands of the mask, both rows
};

// Query side of the mask step: bf16 k slots [0, 0, 0, 1, 1, 1, 0, 0] in lanes
// 0..31 and zero in lanes 32..63; against the key side [1, 1, 1, m, m, m, 0, 0]
// (m = sqrt(d) * mask split in three) it adds sqrt(d) * mask.
__device__ __forceinline__ u32x4 mask_query_side(int lane) {
  const u32x4 v = {0u, pipe::kBf16One << 16, pipe::kBf16One | (pipe::kBf16One << 16), 0u};
  return (lane >> 5) ? u32x4{0u, 0u, 0u, 0u} : v;
}

// One unit of work: one head, one pair of attention rows (r0, r1; r1 == r0 when
// the pair has one row) and one block of 128 queries.  Its keys are visited in
// nb >= 2 blocks of 64 (up to the last key that is live in either row; at least
// two blocks, so that the copies two blocks ahead never reach past the next
// item; blocks past the keys hold -inf bias and contribute nothing).
struct FwdItem {
  int h, qb, r0, r1;
  bool v1;
  int live0, live1;  // last live key of each row (N - 1 without a mask, -1 if none)
  int nb;
  int brow;          // tile index (h nt + qt) nt of the bias tile (this wave's query tile qt, key tile 0)
  int64_t o0, o1;    // element offsets of (r0, position 0, h) and (r1, position 0, h)
};

template <int D, bool MASKED>
__global__ __launch_bounds__(256, 2) void fwd_pp_kernel(Problem p, FwdArgs a, const float* __restrict__ bias_t,
                                                        const u32x4* __restrict__ kaug,
                                                        const int* __restrict__ last_live, int nt) {
  constexpr int TB = Tile<D>::BYTES;
  constexpr int KS = Shape<D>::KS;
  static_assert(Shape<D>::DB == 1, "head_dim <= 32");
  using St = dma::Stager<D, 4>;
  __shared__ __align__(16) FwdStage<D> sm0, sm1, sm2, sm3;
  __shared__ __align__(16) uint32_t zero16[4];
  if (threadIdx.x < 4) zero16[threadIdx.x] = 0u;  // (published by the prologue's barrier)

  const int nqb = (p.N + kPpQueries - 1) / kPpQueries;
  const int nrg = (p.R + 1) / 2;
  const int nkb = (p.N + kBlk - 1) / kBlk;
  const int wave = pipe::wave_id(), lane = threadIdx.x & 63, half = lane >> 5;
  // log2(e) / sqrt(d) as a compile-time constant: the logit FMA below then takes it
  // as an instruction literal (a two-operand encoding that issues faster).
  static_assert(D == 8 || D == 16 || D == 32, "head_dim");
  constexpr float c1 = D == 8 ? kLog2e * 0.35355339059327376f : D == 16 ? kLog2e * 0.25f : kLog2e * 0.17677669529663687f;
  const uint16_t* const qp = static_cast<const uint16_t*>(a.q);
  const uint16_t* const kp = static_cast<const uint16_t*>(a.k);
  const uint16_t* const vp = static_cast<const uint16_t*>(a.v);

  // Items of this workgroup.  Workgroup w runs on XCD w % 8; the XCD owns one
  // contiguous range of items (neighbouring items share a row pair's K and V
  // and a head's bias in that XCD's L2) and its workgroups take every Sx-th.
  const int total = nqb * nrg * p.H;
  const int G = gridDim.x, xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int Sx = (G - xcd + 7) >> 3;
  const int q8 = total >> 3, rem8 = total & 7;
  const int lo = xcd * q8 + min(xcd, rem8);
  const int hi = lo + q8 + (xcd < rem8 ? 1 : 0);
  int next_index = lo + slot;  // index of the next item to set up

  auto make_item = [&](int i) __attribute__((always_inline)) -> FwdItem {
    FwdItem it;
    it.qb = i % nqb;
    const int t = i / nqb;
    const int rg = t % nrg;
    it.h = t / nrg;
    it.r0 = 2 * rg;
    it.v1 = 2 * rg + 1 < p.R;
    it.r1 = it.v1 ? 2 * rg + 1 : 2 * rg;
    if constexpr (MASKED) {
      it.live0 = last_live[it.r0];
      it.live1 = last_live[it.r1];
    } else {
      it.live0 = it.live1 = p.N - 1;
    }
    const int n_eff = min(p.N, (max(it.live0, it.live1) + kBlk) / kBlk * kBlk);
    it.nb = max(2, (n_eff + kBlk - 1) / kBlk);
    it.brow = (it.h * nt + min(it.qb * (kPpQueries / 32) + wave, nt - 1)) * nt;
    it.o0 = row_head_offset(p, it.r0, it.h);
    it.o1 = row_head_offset(p, it.r1, it.h);
    return it;
  };
  auto item_j = [&](const FwdItem& it) __attribute__((always_inline)) {
    return it.qb * kPpQueries + wave * 32 + (lane & 31);
  };
  // Slabs of K and V of both rows: K r0, V r0, K r1, V r1.
  auto slabs = [&](const FwdItem& it, const char* (&b)[4]) __attribute__((always_inline)) {
    b[0] = reinterpret_cast<const char*>(kp + it.o0);
    b[1] = reinterpret_cast<const char*>(vp + it.o0);
    b[2] = reinterpret_cast<const char*>(kp + it.o1);
    b[3] = reinterpret_cast<const char*>(vp + it.o1);
  };
  auto load_q = [&](const FwdItem& it, u32x4 (&dst)[2][KS]) __attribute__((always_inline)) {
    const int j = item_j(it);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      dst[0][ks] = global_operand<D>(p, qp, it.r0, j, it.h, ks, half);
      dst[1][ks] = global_operand<D>(p, qp, it.r1, j, it.h, ks, half);
    }
    if constexpr (D == 8 && MASKED) {
      // k slots 8..15 (lanes 32..63) carry the query side of the mask step.
      if (half) dst[0][0] = dst[1][0] = mask_query_side(0);
    }
  };

  St st;
  st.init(wave, lane, static_cast<uint32_t>(p.pos_stride * p.H * D * 2));
  Reads<D> rd;
  rd.init(lane);
  const u32x4 mq = mask_query_side(lane);

  auto stage = [&](auto sc) __attribute__((always_inline)) -> FwdStage<D>& {
    constexpr int s = decltype(sc)::value;
    if constexpr (s == 0) return sm0;
    else if constexpr (s == 1) return sm1;
    else if constexpr (s == 2) return sm2;
    else return sm3;
  };

  // The stream of key blocks: the current item covers global blocks
  // [gb_cur, gb_nxt), the next one (if any) starts at gb_nxt.
  FwdItem cur = make_item(next_index);
  next_index += Sx;
  const bool first_has_next = next_index < hi;
  FwdItem nxt = cur;
  bool has_nxt = first_has_next;
  if (has_nxt) nxt = make_item(next_index);
  int gb_cur = 0;
  int gb_nxt = cur.nb;

  // Item and local block of global block gb (gb < gb_nxt + 2); a block past the
  // last item resolves to the current item's last block (copied, never used).
  auto resolve = [&](int gb, FwdItem& it, int& lb) __attribute__((always_inline)) {
    if (gb < gb_nxt) {
      it = cur;
      lb = gb - gb_cur;
    } else if (has_nxt) {
      it = nxt;
      lb = gb - gb_nxt;
    } else {
      it = cur;
      lb = cur.nb - 1;
    }
  };
  // Copies of global block gb into stage sc: K, V of both rows, and the mask
  // operands (waves 0, 2 copy row 0's, waves 1, 3 row 1's: the same bytes twice).
  auto issue_copies = [&](int gb, auto sc) __attribute__((always_inline)) {
    FwdItem it;
    int lb;
    resolve(gb, it, lb);
    const int b = min(lb, nkb - 1);
    FwdStage<D>& sg = stage(sc);
    const char* base[4];
    slabs(it, base);
    st.issue(lds_ptr(sg.kv), base, b * kBlk, p.N, wave);
    if constexpr (MASKED) {
      const u32x4* row = kaug + static_cast<int64_t>((wave & 1) ? it.r1 : it.r0) * p.N;
      lds_char* dst = lds_ptr(sg.kaug) + (wave & 1) * kBlk * 16;
      if (b * kBlk + kBlk <= p.N)
        copy16(pipe::uniform_ptr(row + b * kBlk), static_cast<uint32_t>(lane) * 16, dst);
      else
        copy16(row + min(b * kBlk + lane, p.N - 1), dst);
    }
  };
  // sqrt(d) * bias of this wave's 32 queries for global tile gt (of global block
  // gt / 2); tiles past the keys read the item's last tile column.
  auto load_bias = [&](f32x16& dst, int gt) __attribute__((always_inline)) {
    FwdItem it;
    int lb;
    resolve(gt >> 1, it, lb);
    const int kt = min(2 * lb + (gt & 1), nt - 1);
    dst = load_tile_acc(bias_t + static_cast<int64_t>(it.brow + kt) * 1024, lane);  // 1024 floats per tile
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  using I4 = std::integral_constant<int, 4>;
  using I5 = std::integral_constant<int, 5>;
  using I6 = std::integral_constant<int, 6>;
  using I7 = std::integral_constant<int, 7>;
  using True = std::true_type;
  using False = std::false_type;

  u32x4 qreg[2][KS], qnext[2][KS];
  f32x16 S[2], O[2], bias[4];
  u32x4 P[2][2];
  float nm_run[2], l_run[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int e = 0; e < 16; ++e) O[i][e] = 0.f;
    nm_run[i] = 0.f;  // minus the reference point of this query's exponentials, log2 units
    l_run[i] = 0.f;  // this lane's share of the running sum
  }

  // MFMA operands of a half-step, read from LDS at its start: V^T of the tile
  // whose P V product it forms, K and the mask operand of the tile whose logits
  // it forms.
  struct Ops {
    u32x4 v[2], k[KS], ka;
  };
  Ops ops;
  auto read_v = [&](auto i_c, auto sc, auto tib_c) __attribute__((always_inline)) {
    constexpr int i = decltype(i_c)::value;
    constexpr int TIB = decltype(tib_c)::value;
    lds_char* vt = lds_ptr(stage(sc).kv) + (2 * i + 1) * TB;
    ops.v[0] = rd.tr_operand(vt, 0, 32 * TIB, 0);
    ops.v[1] = rd.tr_operand(vt, 0, 32 * TIB, 1);
  };
  auto read_k = [&](auto i_c, auto sc, auto tib_c) __attribute__((always_inline)) {
    constexpr int i = decltype(i_c)::value;
    constexpr int TIB = decltype(tib_c)::value;
    lds_char* kt = lds_ptr(stage(sc).kv) + (2 * i) * TB;
    if constexpr (D == 8 && MASKED) {
      // At d = 8 the mask operand rides in k slots 8..15 (lanes 32..63) of the
      // logits' one MFMA step.
      const u32x4 kv = ld16(kt + rd.rows[0] + 32 * TIB * (2 * D));
      const u32x4 ka = ld16(lds_ptr(stage(sc).kaug) + (i * kBlk + 32 * TIB + (lane & 31)) * 16);
      ops.k[0] = half ? ka : kv;
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) ops.k[ks] = rd.rows_operand(kt, 32 * TIB, ks, lane);
      // (lanes 32..63 hold k slots 8..15, zero on the query side: they read 16 zero
      // bytes, since a masked key's operand holds -inf)
      if constexpr (MASKED)
        ops.ka = ld16(half ? lds_ptr(zero16) : lds_ptr(stage(sc).kaug) + (i * kBlk + 32 * TIB + (lane & 31)) * 16);
    }
  };
  // Logits of row I for the tile in ops into S[I] (accumulator input c = bias).
  auto logits = [&](auto i_c, const f32x16& c) __attribute__((always_inline)) {
    constexpr int i = decltype(i_c)::value;
    f32x16 acc = mma(ops.k[0], qreg[i][0], c);
#pragma unroll
    for (int ks = 1; ks < KS; ++ks) acc = mma(ops.k[ks], qreg[i][ks], acc);
    if constexpr (MASKED && D != 8) acc = mma(ops.ka, mq, acc);
    S[i] = acc;
  };
  // O^T of row I += V^T P^T for the tile in ops.
  auto pv = [&](auto i_c) __attribute__((always_inline)) {
    constexpr int i = decltype(i_c)::value;
    O[i] = mma(ops.v[0], P[i][0], O[i]);
    O[i] = mma(ops.v[1], P[i][1], O[i]);
  };
  // Probabilities of row I's tile in S[I] against reference point m (log2
  // units): P[I] (bf16) and the fp32 sum of this lane's 16 terms.
  auto exponentiate = [&](auto i_c, float mneg) __attribute__((always_inline)) -> float {
    constexpr int i = decltype(i_c)::value;
    float pr[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) pr[e] = fast_exp2(__builtin_fmaf(S[i][e], c1, mneg));
    float ls[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) ls[c] = (pr[c] + pr[c + 4]) + (pr[c + 8] + pr[c + 12]);
#pragma unroll
    for (int u = 0; u < 2; ++u)
      P[i][u] = u32x4{pack_bf16(pr[8 * u + 0], pr[8 * u + 1]), pack_bf16(pr[8 * u + 2], pr[8 * u + 3]),
                      pack_bf16(pr[8 * u + 4], pr[8 * u + 5]), pack_bf16(pr[8 * u + 6], pr[8 * u + 7])};
    return (ls[0] + ls[1]) + (ls[2] + ls[3]);
  };
  // Scheduling of a half-step: its LDS operand reads first, then a first share
  // of the softmax's vector work (it depends only on the previous half-step's
  // logits, so it covers the LDS latency), then each MFMA followed by a share of
  // the vector work.
  auto schedule_half_step = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_group_barrier(0x100, 12, 0);  // LDS reads
    __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);  // vector ALU
#pragma unroll
    for (int m = 0; m < 5; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);  // vector ALU
    }
  };
  // Online softmax of row I's tile.  The reference point starts at 0 and moves
  // only when the running sum leaves [2^-64, 2^64]: then every probability and
  // the sums stay far inside the fp32 and bf16 range.  On a move the point goes
  // to the running maximum (to the tile's maximum while nothing has been summed
  // yet, so it may also go down) and O, l are rescaled.
  auto softmax = [&](auto i_c) __attribute__((always_inline)) {
    constexpr int i = decltype(i_c)::value;
    float lsum = exponentiate(i_c, nm_run[i]);
    const uint32_t lb = __float_as_uint(l_run[i] + lsum) - 0x1F800000u;  // 2^-64
    schedule_half_step();
    if (__builtin_expect(__ballot(!(lb < 0x40000000u)) != 0, 0)) {       // 2^64 / 2^-64
      float mx = S[i][0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mx = fmaxf(mx, S[i][e]);
      mx = pair_max(mx) * c1;
      const bool empty = pair_sum(l_run[i]) == 0.f;
      const float m_new = empty ? mx : fmaxf(-nm_run[i], mx);
      const float alpha = empty || m_new == -INFINITY ? 0.f : fast_exp2(-nm_run[i] - m_new);
      l_run[i] *= alpha;
#pragma unroll
      for (int e = 0; e < 16; ++e) O[i][e] *= alpha;
      nm_run[i] = -m_new;
      lsum = exponentiate(i_c, m_new == -INFINITY ? 0.f : -m_new);  // (no live key yet: every p is 0)
    }
    l_run[i] += lsum;
  };
  // Normalised O and the natural-log lse of row I of item it; the row's state is
  // reset for the next item.
  auto finalize = [&](auto i_c, const FwdItem& it) __attribute__((always_inline)) {
    constexpr int i = decltype(i_c)::value;
    const float l_tot = pair_sum(l_run[i]);
    const int j = item_j(it);
    const int r = i ? it.r1 : it.r0;
    const bool dead = (i ? it.live1 : it.live0) < 0 || !(l_tot > 0.f);  // every key of the row masked
    const float inv = dead ? 0.f : 1.f / l_tot;
    if (j < p.N && (i == 0 || it.v1)) {
      if constexpr (D >= 16)
        store_dT_x16<D>(static_cast<uint16_t*>(a.o) + elem_offset(p, r, j, it.h), O[i], inv, half);
      else
        store_dT<D>(static_cast<uint16_t*>(a.o) + elem_offset(p, r, j, it.h), &O[i], inv, half);
      if (a.lse && half == 0)
        a.lse[(static_cast<int64_t>(r) * p.H + it.h) * p.N + j] =
            dead ? -INFINITY : (__log2f(l_tot) - nm_run[i]) * kLn2;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) O[i][e] = 0.f;
    nm_run[i] = 0.f;
    l_run[i] = 0.f;
  };

  // Half-step A of global tile g (phase PH = g % 8): row 1's P V of tile g - 1
  // and logits of tile g on the matrix cores beside row 0's softmax of tile g on
  // the vector ALU.  After the second tile of global block b the copies and bias
  // loads issued one block earlier are retired (the compiler's own wait for bias
  // registers would drain every outstanding vector memory operation, so each
  // block's global traffic is issued at known points): block b + 1's stage and
  // the bias of its tiles have arrived; the bias of block b + 2's tiles starts
  // (its copies half a step later, in half-step B, which spreads the
  // vector-memory issue over the block).  After the current item's last tile row 0 switches to the next
  // item's queries (its logits of the next tile belong to the next item).
  auto half_a = [&](int g, auto ph_c, auto first_c) __attribute__((always_inline)) {
    constexpr int PH = decltype(ph_c)::value;
    constexpr bool FIRST = decltype(first_c)::value;
    constexpr int S_T = (PH / 2) % 4, TIB_T = PH % 2;
    constexpr int S_P = (((PH + 7) % 8) / 2) % 4, TIB_P = (PH + 7) % 2;
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!FIRST) read_v(I1(), std::integral_constant<int, S_P>(), std::integral_constant<int, TIB_P>());
    read_k(I1(), std::integral_constant<int, S_T>(), std::integral_constant<int, TIB_T>());
    if constexpr (!FIRST) pv(I1());
    logits(I1(), bias[PH % 4]);
    softmax(I0());
    if constexpr (PH % 2 == 1) {
      wait_vm<0>();
      lds_barrier();
      load_bias(bias[(PH + 3) % 4], g + 3);
      load_bias(bias[(PH + 4) % 4], g + 4);
      if (g == 2 * gb_nxt - 1) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qreg[0][ks] = qnext[0][ks];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // Half-step B of global tile g: row 0's P V of tile g and logits of tile g + 1
  // beside row 1's softmax of tile g.  After the current item's last tile row 0
  // of the item is complete, and row 1 switches to the next item's queries.
  auto half_b = [&](int g, auto ph_c) __attribute__((always_inline)) {
    constexpr int PH = decltype(ph_c)::value;
    constexpr int S_T = (PH / 2) % 4, TIB_T = PH % 2;
    constexpr int S_N = (((PH + 1) % 8) / 2) % 4, TIB_N = (PH + 1) % 2;
    __builtin_amdgcn_sched_barrier(0);
    read_v(I0(), std::integral_constant<int, S_T>(), std::integral_constant<int, TIB_T>());
    read_k(I0(), std::integral_constant<int, S_N>(), std::integral_constant<int, TIB_N>());
    pv(I0());
    logits(I0(), bias[(PH + 1) % 4]);
    softmax(I1());
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (PH % 2 == 1) {
      // The copies of block b + 2 (into the stage of block b - 2, long free).
      issue_copies((g + 1) / 2 + 1, std::integral_constant<int, ((PH + 1) / 2 + 1) % 4>());
      if (g == 2 * gb_nxt - 1) {
        finalize(I0(), cur);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qreg[1][ks] = qnext[1][ks];
      }
    }
  };
  // After half-step A of the first tile of an item: row 1 of the previous item is
  // complete; the next item becomes current and the one after it is set up (its
  // queries are loaded now, long before they are needed).
  auto advance = [&](int g) __attribute__((always_inline)) {
    if (g == 2 * gb_nxt) {
      finalize(I1(), cur);
      cur = nxt;
      gb_cur = gb_nxt;
      gb_nxt = gb_cur + cur.nb;
      next_index += Sx;
      has_nxt = next_index < hi;
      if (has_nxt) {
        nxt = make_item(next_index);
        load_q(nxt, qnext);
      }
    }
  };

  // Prologue: the first item's queries and the bias of its tiles 0..3, the next
  // item's queries, the copies of blocks 0 and 1, all retired before row 0's
  // first logits.
  load_q(cur, qreg);
  if (first_has_next) load_q(nxt, qnext);
#pragma unroll
  for (int t = 0; t < 4; ++t) load_bias(bias[t], t);
  issue_copies(0, I0());
  issue_copies(1, I1());
  wait_vm<0>();
  lds_barrier();
  read_k(I0(), I0(), I0());
  logits(I0(), bias[0]);
  half_a(0, I0(), True());
  int g = 0;
  for (;; g += 8) {
    half_b(g, I0());
    if (g == 2 * gb_nxt - 1 && !has_nxt) break;
    half_a(g + 1, I1(), False());
    half_b(g + 1, I1());
    if (g + 1 == 2 * gb_nxt - 1 && !has_nxt) { g += 1; break; }
    half_a(g + 2, I2(), False());
    advance(g + 2);
    half_b(g + 2, I2());
    if (g + 2 == 2 * gb_nxt - 1 && !has_nxt) { g += 2; break; }
    half_a(g + 3, I3(), False());
    half_b(g + 3, I3());
    if (g + 3 == 2 * gb_nxt - 1 && !has_nxt) { g += 3; break; }
    half_a(g + 4, I4(), False());
    advance(g + 4);
    half_b(g + 4, I4());
    if (g + 4 == 2 * gb_nxt - 1 && !has_nxt) { g += 4; break; }
    half_a(g + 5, I5(), False());
    half_b(g + 5, I5());
    if (g + 5 == 2 * gb_nxt - 1 && !has_nxt) { g += 5; break; }
    half_a(g + 6, I6(), False());
    advance(g + 6);
    half_b(g + 6, I6());
    if (g + 6 == 2 * gb_nxt - 1 && !has_nxt) { g += 6; break; }
    half_a(g + 7, I7(), False());
    half_b(g + 7, I7());
    if (g + 7 == 2 * gb_nxt - 1 && !has_nxt) { g += 7; break; }
    half_a(g + 8, I0(), False());
    advance(g + 8);
  }
  // Row 1's P V of the last tile g (every copy retired first: the stage is
  // chosen at run time), then its row of the last item.
  wait_vm<0>();
  switch ((g / 2) % 4 * 2 + g % 2) {
    case 0: read_v(I1(), I0(), I0()); break;
    case 1: read_v(I1(), I0(), I1()); break;
    case 2: read_v(I1(), I1(), I0()); break;
    case 3: read_v(I1(), I1(), I1()); break;
    case 4: read_v(I1(), I2(), I0()); break;
    case 5: read_v(I1(), I2(), I1()); break;
    case 6: read_v(I1(), I3(), I0()); break;
    default: read_v(I1(), I3(), I1()); break;
  }
  pv(I1());
  finalize(I1(), cur);
}

}  // namespace

// Compute units of the current device (cached per device).
int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

namespace {

template <int D>
hipError_t fwd_pp_dispatch(const Problem& p, const FwdArgs& a, float* bias_t, u32x4* kaug, int* last_live,
                           hipStream_t s) {
  hipError_t e = launch_fwd_prep(p, a.bias, a.mask, bias_t, kaug, last_live, s);
  if (e != hipSuccess) return e;
  // Persistent workgroups: two per compute unit (their LDS and registers allow
  // two), each working through its share of the items.
  const int64_t items = static_cast<int64_t>((p.N + kPpQueries - 1) / kPpQueries) * p.H * ((p.R + 1) / 2);
  const int64_t blocks = std::min<int64_t>(items, 2 * static_cast<int64_t>(device_cus()));
  const int nt = bias_tiles(p.N);
  KernelTimer timer("fwd_mfma", s);
  if (a.mask)
    hipLaunchKernelGGL((fwd_pp_kernel<D, true>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p, a, bias_t,
                       kaug, last_live, nt);
  else
    hipLaunchKernelGGL((fwd_pp_kernel<D, false>), dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p, a, bias_t,
                       kaug, last_live, nt);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_pp(const Problem& p, const FwdArgs& a, float* bias_t, void* kaug, int* last_live,
                         hipStream_t s) {
  u32x4* ka = static_cast<u32x4*>(kaug);
  switch (p.D) {
    case 8: return fwd_pp_dispatch<8>(p, a, bias_t, ka, last_live, s);
    case 16: return fwd_pp_dispatch<16>(p, a, bias_t, ka, last_live, s);
    case 32: return fwd_pp_dispatch<32>(p, a, bias_t, ka, last_live, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace evo
