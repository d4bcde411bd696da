// Weight-streaming grouped expert GEMMs (gate/up + SwiGLU, and down) for the
// decode regime, where every expert sees only a few dozen rows and the time
// goes into reading each expert's weights once from HBM.  Experts are large,
// sparsely activated matrix products (A/F 分离 page, "为什么要拆"); at
// decode batch sizes their cost is the weight bytes.
//
// Design (gfx950, wave64):
//  * Persistent workgroups claim work items (row tile x column tile) from a
//    device counter that the dispatch kernel zeroes, so the grid never
//    depends on host-side counts and the tail is one item long.
//  * Each wave owns 16 weight rows of each matrix (gate and up, or down).
//    Weights go from global memory straight into MFMA operand registers,
//    one "super-stage" (SS bytes of K per row) ahead of the math: no LDS
//    round trip and no barrier on the weight path.  Load instruction i of a
//    super-stage reads bytes [64 i, 64 i + 64) of 16 rows (lane group
//    q = lane/16 takes 16 bytes at 64 i + 16 q), so every instruction moves
//    whole 64-byte row segments.
//  * The gathered activation rows (a few KB per tile, shared by all waves)
//    are staged through LDS, double-buffered per super-stage.  The down
//    GEMMs and the 128-row fp8 gate/up GEMM load them (and in fp8 the
//    scales the store needs) two super-stages ahead, so that storing them
//    to LDS never waits on a load issued in the same stage; the bf16
//    gate/up shapes load them one stage ahead (the second slot spills
//    there).  The bf16 128-row shapes stage only the passes a tile's rows
//    fill and, when that is half or a quarter of them, load two stages
//    ahead with the registers saved.
//  * bf16: chunk i is one 16x16x32 MFMA.  fp8: chunks 2b and 2b+1 (bytes
//    [128 b + 16 q] and [128 b + 64 + 16 q]) lie in the same 128-wide K
//    block b and feed one 16x16x128 MFMA; the block's partial sum is then
//    scaled by (activation scale of the row) x (weight block scale), a
//    product staged once per row and block in LDS.  A and B use the same
//    byte->K assignment, so the products are exact permutations of the K
//    sum.
//  * Every load of the main loop is unconditional and issued A rows, A
//    scale, B scales, B rows (the last stage is peeled): vector loads
//    complete in order, so the wait before the A store leaves the next
//    stage's weights in flight, and no branch makes the compiler's wait
//    before an MFMA cover loads just issued.
//  * Epilogues stage the tile through LDS and write whole 16-byte pieces.
//    The fp8 gate/up epilogue of a 128-column item (one 1x128 quantisation
//    group) writes E4M3 z and its scales; a 64-column item writes fp32 z
//    for the standalone quantiser.
#include "common.h"
#include <atomic>
#include <type_traits>

#include "kernels.h"

namespace afd {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + expf(-g)) * u;
}

// WIDE (bf16 down only): an item covers two blocks of BN output columns,
// held like the gate and up blocks of a gate/up item (two weight-row blocks
// per wave, one staged activation tile for both).
template <Elem EL, int WAVES, int BM, int SS, bool SWIGLU, bool WIDE = false>
struct StreamCfg {
  static constexpr int kThreads = WAVES * 64;
  static constexpr int NMAT = SWIGLU || WIDE ? 2 : 1;
  static constexpr int BN = 16 * WAVES;       // columns per matrix per item
  static constexpr int ICOLS = WIDE ? 2 * BN : BN;  // output columns per item
  static constexpr int MB = BM / 16;
  static constexpr int NPR = SS / 128;        // 128-byte K pieces per row per super-stage
  static constexpr int APITCH = SS + 16;      // LDS row pitch of the A stage
  static constexpr int CPR = SS / 16;         // 16-byte chunks of one A row per super-stage
  static constexpr int RPP = kThreads / CPR;  // A rows staged per pass of the workgroup
  static constexpr int RA = BM / RPP;         // passes
  static constexpr int KB = SS / 128;         // fp8 scale blocks per super-stage
  static constexpr bool FP8 = EL == Elem::FP8;
  static constexpr int LDS_A = 2 * BM * APITCH;
  // epilogue staging: BM rows x BN columns of the output element
  static constexpr int OUT_ES = FP8 && SWIGLU ? 4 : 2;  // fp32 z (W8A8) or bf16
  static constexpr int LDS_OUT = BM * ICOLS * OUT_ES;
  static constexpr int LDS = LDS_A > LDS_OUT ? LDS_A : LDS_OUT;
  // fp8: activation scale x weight block scale, [buffer][matrix][K block][row]
  using SAs = float[2][NMAT][FP8 ? KB : 1][FP8 ? BM : 4];
  static_assert(BM % 16 == 0 && SS % 128 == 0, "shape");
  static_assert(kThreads % CPR == 0 && BM % RPP == 0, "A staging passes");
  static_assert(!FP8 || 128 % BN == 0, "fp8: an item lies inside one weight scale block row");
  static_assert(!FP8 || BM * KB <= kThreads, "fp8: one activation scale per thread");
  static_assert(!WIDE || (!SWIGLU && !FP8), "wide items: bf16 down GEMM only");
};

// Synchronisation of an item with the other GEMM of the same forward, for
// the single launch that runs both weight-streaming GEMMs (gate/up items
// first, then down items, from one work counter):
//  kNoSync: the GEMM runs on its own (one launch per GEMM);
//  kSignal: a gate/up item writes its z columns through to memory
//           (agent-scope stores) and then counts itself finished in the
//           tile's counter;
//  kWait:   a down item waits until every gate/up item of its tile has
//           counted itself (a bounded wait) before it reads z.
// The launch's sync words: sync[0] counts down items that gave up waiting,
// sync[1 + t] is the counter of tile t.
enum { kNoSync = 0, kSignal = 1, kWait = 2 };

// Polls of a tile counter before a down item gives up waiting (about a
// quarter of a second; a legitimate wait is one gate/up item, a few hundred
// microseconds).  Every gate/up item is claimed before any down item, by a
// workgroup that is running and waits on nothing, so the bound is never
// reached; it only keeps a defect from hanging the device, and such an item
// is counted in sync[0], which the traced forward reports.
constexpr int kTileWaitPolls = 1 << 18;

// 16-byte store that is visible to every CU of the device once the store
// counter has drained (two agent-scope 8-byte stores).
__device__ __forceinline__ void st16_agent(uint8_t *dst, u32x4 v) {
  uint64_t *d = reinterpret_cast<uint64_t *>(dst);
  __hip_atomic_store(d, static_cast<uint64_t>(v[0]) | (static_cast<uint64_t>(v[1]) << 32),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(d + 1, static_cast<uint64_t>(v[2]) | (static_cast<uint64_t>(v[3]) << 32),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// K (in bytes per row) must be a multiple of SS for every group; the
// launcher picks an instantiation that satisfies this, so the main loop has
// no partial super-stage and no per-load guard.
// AD: how many super-stages ahead the activation rows are loaded (1 or 2).
// One work item (row tile x BN columns) of the weight-streaming GEMM.
// sync / GU_BN: the sync words (see kNoSync) and the gate/up item width of
// the single launch (SYNC != kNoSync).
template <Elem EL, int WAVES, int BM, int SS, bool SWIGLU, int AD, int SYNC, int GU_BN = 0,
          bool WIDE = false>
__device__ __forceinline__ void stream_item(
    const GemmArgs &p, const int item, uint8_t *lds,
    typename StreamCfg<EL, WAVES, BM, SS, SWIGLU, WIDE>::SAs &sAs, int32_t *sync) {
  using C = StreamCfg<EL, WAVES, BM, SS, SWIGLU, WIDE>;
  constexpr int ICOLS = C::ICOLS;
  constexpr int NMAT = C::NMAT, BN = C::BN, MB = C::MB, NPR = C::NPR;
  constexpr int APITCH = C::APITCH, CPR = C::CPR, RPP = C::RPP, RA = C::RA, KB = C::KB;
  static_assert(AD == 1 || AD == 2, "activation prefetch distance");
  static_assert(SYNC == kNoSync || (!C::FP8 && (SYNC != kSignal || SWIGLU) &&
                                    (SYNC != kWait || (!SWIGLU && GU_BN > 0))),
                "the single launch of both GEMMs is bf16: gate/up signals, down waits");

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, r16 = lane & 15;
  const int nmax = p.N > p.Ns ? p.N : p.Ns;
  const int ntn = nmax / ICOLS;
  const int acol = tid % CPR, arow0 = tid / CPR;  // this thread's A chunk column, first row
  constexpr int ES = C::FP8 ? 1 : 2;

  {
    const int ti = item / ntn;
    const Tile tile = p.tiles[ti];
    const int nt = item % ntn;
    const bool shared = tile.group >= p.E;
    const int N = shared ? p.Ns : p.N;
    const int K = shared ? p.Ks : p.K;
    const int n0 = nt * ICOLS;
    if (n0 >= N) return;  // uniform over the workgroup
    const int g = shared ? tile.group - p.E : tile.group;
    const int rows = tile.rows;
    const int64_t krow = static_cast<int64_t>(K) * ES;
    const int nss = static_cast<int>(krow / SS);

    if constexpr (SYNC == kWait) {
      // z of this tile is complete once its K / GU_BN gate/up items (the
      // down GEMM's K is the gate/up GEMM's N) have counted themselves
      if (tid == 0) {
        const int need = K / GU_BN;
        bool ready = false;
        for (int poll = 0; poll < kTileWaitPolls && !ready; ++poll) {
          ready = __hip_atomic_load(sync + 1 + ti, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= need;
          if (!ready) __builtin_amdgcn_s_sleep(2);
        }
        if (!ready) __hip_atomic_fetch_add(sync, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();
    }

    // A rows this thread stages; rows past the tile's end repeat its first
    // row (they only feed output rows that are never stored)
    auto source_row = [&](int row) {
      const int r = tile.row0 + (row < rows ? row : 0);
      return p.perm ? (r < p.Tk ? p.perm[r] : (r - p.Tk) % p.T) : r;
    };
    // The item body, for RAX staging passes of the A rows (the passes that
    // hold rows of this tile) and activation prefetch distance ADX.  Tiles
    // that fill half or a quarter of the passes stage only those and, with
    // the staging registers that frees, load the rows two stages ahead.
    auto body = [&](auto rax_c, auto adx_c) {
      constexpr int RAX = decltype(rax_c)::value;
      constexpr int ADX = decltype(adx_c)::value;
      // the staged rows cover every active 16-row MFMA block
      static_assert((RAX * RPP) % 16 == 0, "staged rows are whole row blocks");
      int asrc[RAX];
  #pragma unroll
      for (int i = 0; i < RAX; ++i) asrc[i] = source_row(arow0 + i * RPP);
      const uint8_t *abase_g = p.A + acol * 16;
      // activation scales: thread tid < BM * KB stages scale (row tid / KB,
      // block tid % KB); the others load a valid address and drop the value,
      // so every load of the main loop is unconditional
      const float *asc = p.a_scale;
      if constexpr (C::FP8) {
        const int as_t = tid < BM * KB ? tid : 0;
        asc = p.a_scale + static_cast<int64_t>(source_row(as_t / KB)) * p.a_scale_pitch + as_t % KB;
      }

      const int64_t mat = static_cast<int64_t>(N) * krow;
      const uint8_t *bptr[NMAT];
      {
        const uint8_t *b0 = (shared ? p.sb0 : p.b0) + g * mat;
        bptr[0] = b0 + static_cast<int64_t>(n0 + wave * 16 + r16) * krow + q * 16;
        if constexpr (SWIGLU) {
          const uint8_t *b1 = (shared ? p.sb1 : p.b1) + g * mat;
          bptr[NMAT - 1] = b1 + static_cast<int64_t>(n0 + wave * 16 + r16) * krow + q * 16;
        } else if constexpr (WIDE) {
          bptr[1] = b0 + static_cast<int64_t>(n0 + BN + wave * 16 + r16) * krow + q * 16;
        }
      }
      const float *bsc[NMAT] = {};
      if constexpr (C::FP8) {
        const int kblocks = K / 128;
        const int64_t sblk = static_cast<int64_t>(N / 128) * kblocks;
        bsc[0] = (shared ? p.sbs0 : p.bs0) + g * sblk + (n0 / 128) * kblocks;
        if constexpr (SWIGLU) bsc[NMAT - 1] = (shared ? p.sbs1 : p.bs1) + g * sblk + (n0 / 128) * kblocks;
      }
      const int mb_active = (rows + 15) >> 4;

      // ---- registers: 128-byte K piece c of a row block is one 8-dword tuple
      // (bytes [128 c + 16 q] and [128 c + 64 + 16 q]), one fp8 MFMA operand or
      // two bf16 MFMA operands
      u32x8 bq[2][NMAT][NPR];
      // what the LDS store of ADX super-stages needs, slot = stage % ADX:
      // activation rows, and in fp8 the activation scale and the B block
      // scales (the store writes their product)
      u32x4 ra[ADX][RAX];
      float as_reg[ADX] = {};
      float sbs[ADX][NMAT][C::FP8 ? KB : 1];
      // order of issue: A rows, A scale, B scales, then the B rows of a stage.
      // Vector loads complete in order, so a wait for the first three leaves
      // the B rows issued after them in flight.
      auto load_a = [&](auto slot_c, int ss) {
        constexpr int SL = decltype(slot_c)::value;
  #pragma unroll
        for (int i = 0; i < RAX; ++i)
          ra[SL][i] = ld16(abase_g + static_cast<int64_t>(asrc[i]) * p.a_pitch +
                           static_cast<int64_t>(ss) * SS);
        if constexpr (C::FP8) {
          as_reg[SL] = asc[ss * KB];
  #pragma unroll
          for (int m = 0; m < NMAT; ++m)
  #pragma unroll
            for (int kb = 0; kb < KB; ++kb) sbs[SL][m][kb] = bsc[m][ss * KB + kb];
        }
      };
      auto load_b = [&](u32x8 (&dst)[NMAT][NPR], int ss) {
  #pragma unroll
        for (int m = 0; m < NMAT; ++m)
  #pragma unroll
          for (int c = 0; c < NPR; ++c) {
            const uint8_t *src = bptr[m] + static_cast<int64_t>(ss) * SS + c * 128;
            dst[m][c].lo = ld16(src);
            dst[m][c].hi = ld16(src + 64);
          }
      };
      auto store_a = [&](int buf, auto slot_c) {
        constexpr int SL = decltype(slot_c)::value;
        const float (&sb)[NMAT][C::FP8 ? KB : 1] = sbs[SL];
  #pragma unroll
        for (int i = 0; i < RAX; ++i)
          st16(lds + buf * BM * APITCH + (arow0 + i * RPP) * APITCH + acol * 16, ra[SL][i]);
        if constexpr (C::FP8)
          if (tid < BM * KB) {
            const int kb = tid % KB;
            float sbk[NMAT];
  #pragma unroll
            for (int m = 0; m < NMAT; ++m) {
              // select the block without dynamic register indexing
              float v = sb[m][0];
  #pragma unroll
              for (int k2 = 1; k2 < KB; ++k2) v = kb == k2 ? sb[m][k2] : v;
              sbk[m] = v;
            }
  #pragma unroll
            for (int m = 0; m < NMAT; ++m) sAs[buf][m][kb][tid / KB] = as_reg[SL] * sbk[m];
          }
      };

      f32x4 acc[NMAT][MB];
  #pragma unroll
      for (int m = 0; m < NMAT; ++m)
  #pragma unroll
        for (int b = 0; b < MB; ++b) acc[m][b] = f32x4{0, 0, 0, 0};

      auto compute = [&](const u32x8 (&bb)[NMAT][NPR], int buf) {
        const uint8_t *abase = lds + buf * BM * APITCH + r16 * APITCH + q * 16;
        if constexpr (!C::FP8) {
  #pragma unroll
          for (int b = 0; b < MB; ++b) {
            if (b < mb_active) {
  #pragma unroll
              for (int c = 0; c < NPR; ++c) {
                const u32x4 a0 = ld16(abase + b * 16 * APITCH + c * 128);
                const u32x4 a1 = ld16(abase + b * 16 * APITCH + c * 128 + 64);
  #pragma unroll
                for (int m = 0; m < NMAT; ++m) {
                  acc[m][b] = mfma_bf16_k32(bitcast<bf16x8>(a0), bitcast<bf16x8>(bb[m][c].lo), acc[m][b]);
                  acc[m][b] = mfma_bf16_k32(bitcast<bf16x8>(a1), bitcast<bf16x8>(bb[m][c].hi), acc[m][b]);
                }
              }
            }
            // bound the A reads the compiler hoists to one row block
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
  #pragma unroll
          for (int b = 0; b < MB; ++b) {
            if (b < mb_active) {
  #pragma unroll
              for (int kb = 0; kb < KB; ++kb) {
                u32x8 a;
                a.lo = ld16(abase + b * 16 * APITCH + kb * 128);
                a.hi = ld16(abase + b * 16 * APITCH + kb * 128 + 64);
  #pragma unroll
                for (int m = 0; m < NMAT; ++m) {
                  const f32x4 sab = *reinterpret_cast<const f32x4 *>(&sAs[buf][m][kb][b * 16 + q * 4]);
                  const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                      __builtin_bit_cast(i32x8, a), __builtin_bit_cast(i32x8, bb[m][kb]),
                      f32x4{0, 0, 0, 0}, 0, 0, 0, 127, 0, 127);
  #pragma unroll
                  for (int i = 0; i < 4; ++i) acc[m][b][i] = fmaf(part[i], sab[i], acc[m][b][i]);
                }
              }
            }
            // keep the partial sums of one row block live at a time
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      };

      // ---- pipeline: B one super-stage ahead in registers, A ADX stages ahead
      // in registers and double-buffered in LDS.  The last stage is peeled so
      // that every prefetch in the loop is unconditional: a load behind a
      // branch would make the wait before the next MFMA cover the loads just
      // issued.  With ADX = 2 what is stored after a stage's math was loaded
      // before that stage's weights, so the store never waits on a load issued
      // in the same stage (prefetches past the last stage re-read it).
      using S0 = std::integral_constant<int, 0>;
      using S1 = std::integral_constant<int, ADX - 1>;
      load_a(S0{}, 0);
      if constexpr (ADX == 2) load_a(S1{}, nss > 1 ? 1 : 0);
      load_b(bq[0], 0);
      store_a(0, S0{});
      __syncthreads();
      auto step = [&](auto par, int ss) {  // ss + 1 < nss
        constexpr int P = decltype(par)::value;  // == ss & 1
        if constexpr (ADX == 2) {
          load_a(std::integral_constant<int, P>{}, ss + 2 < nss ? ss + 2 : nss - 1);
          load_b(bq[P ^ 1], ss + 1);
          compute(bq[P], P);
          store_a(P ^ 1, std::integral_constant<int, P ^ 1>{});
        } else {
          load_a(S0{}, ss + 1);
          load_b(bq[P ^ 1], ss + 1);
          compute(bq[P], P);
          store_a(P ^ 1, S0{});
        }
        __syncthreads();
      };
      int ss = 0;
      for (; ss + 2 < nss; ss += 2) {
        step(std::integral_constant<int, 0>{}, ss);
        step(std::integral_constant<int, 1>{}, ss + 1);
      }
      if (ss + 1 < nss) {
        step(std::integral_constant<int, 0>{}, ss);
        compute(bq[1], 1);
      } else {
        compute(bq[0], 0);
      }
      __syncthreads();

      // ---- epilogue (A buffers are free: every wave passed the barrier above)
      if constexpr (SWIGLU && C::FP8) {
        // W8A8: z = silu(g) * u in fp32, staged in LDS
        float *o32 = reinterpret_cast<float *>(lds);
  #pragma unroll
        for (int b = 0; b < MB; ++b)
  #pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = b * 16 + q * 4 + i;
            o32[row * BN + wave * 16 + r16] = silu_mul(acc[0][b][i], acc[1][b][i]);
          }
        __syncthreads();
        if constexpr (BN == 128) {
          // the item is exactly one 1x128 quantisation group wide: four
          // threads per row take 32 columns each, share the row's amax and
          // write E4M3 codes and the group scale (same arithmetic as the
          // standalone quantiser)
          constexpr int TPR = C::kThreads / BM;  // threads per row
          static_assert(TPR * 32 == BN && TPR <= 64 && (64 % TPR) == 0, "row split");
          for (int row = tid / TPR; row < BM; row += C::kThreads / TPR) {
            const int part = tid % TPR;
            const float *src = o32 + row * BN + part * 32;
            float f[32];
  #pragma unroll
            for (int c4 = 0; c4 < 8; ++c4) {
              const u32x4 v = ld16(src + c4 * 4);
  #pragma unroll
              for (int i = 0; i < 4; ++i) f[c4 * 4 + i] = __uint_as_float(v[i]);
            }
            float amax = 0.0f;
  #pragma unroll
            for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(f[i]));
  #pragma unroll
            for (int o = 1; o < TPR; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
            const float sc = e4m3_scale(amax);
            if (row < rows) {
              uint8_t *dst = p.C + static_cast<int64_t>(tile.row0 + row) * p.c_pitch + n0 + part * 32;
  #pragma unroll
              for (int h2 = 0; h2 < 2; ++h2) {
                uint32_t w[4];
  #pragma unroll
                for (int j = 0; j < 4; ++j) {
                  uint32_t word = 0;
  #pragma unroll
                  for (int bb = 0; bb < 4; ++bb)
                    word |= f32_to_e4m3(f[h2 * 16 + j * 4 + bb] / sc) << (8 * bb);
                  w[j] = word;
                }
                st16(dst + h2 * 16, u32x4{w[0], w[1], w[2], w[3]});
              }
              if (part == 0)
                p.c_scale[static_cast<int64_t>(tile.row0 + row) * p.c_scale_pitch + n0 / 128] = sc;
            }
          }
        } else {
          // a quantisation group spans two items: z stays fp32 and the 1x128
          // quantiser runs on it afterwards
          constexpr int PIECES = BM * BN * 4 / 16;
          for (int c = tid; c < PIECES; c += C::kThreads) {
            const int row = c / (BN * 4 / 16), col = c % (BN * 4 / 16);
            if (row < rows)
              st16(p.C + static_cast<int64_t>(tile.row0 + row) * p.c_pitch + n0 * 4 + col * 16,
                   ld16(lds + row * BN * 4 + col * 16));
          }
        }
      } else {
        uint16_t *o16 = reinterpret_cast<uint16_t *>(lds);
  #pragma unroll
        for (int b = 0; b < MB; ++b)
  #pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = b * 16 + q * 4 + i;
            if constexpr (WIDE) {
              o16[row * ICOLS + wave * 16 + r16] = f32_to_bf16(acc[0][b][i]);
              o16[row * ICOLS + BN + wave * 16 + r16] = f32_to_bf16(acc[1][b][i]);
            } else {
              const float v = SWIGLU ? silu_mul(acc[0][b][i], acc[NMAT - 1][b][i]) : acc[0][b][i];
              o16[row * BN + wave * 16 + r16] = f32_to_bf16(v);
            }
          }
        __syncthreads();
        constexpr int PIECES = BM * ICOLS * 2 / 16;
        for (int c = tid; c < PIECES; c += C::kThreads) {
          const int row = c / (ICOLS * 2 / 16), col = c % (ICOLS * 2 / 16);
          if (row < rows) {
            uint8_t *dst = p.C + static_cast<int64_t>(tile.row0 + row) * p.c_pitch + n0 * 2 + col * 16;
            if constexpr (SYNC == kSignal)
              st16_agent(dst, ld16(lds + row * ICOLS * 2 + col * 16));
            else
              st16(dst, ld16(lds + row * ICOLS * 2 + col * 16));
          }
        }
      }
    };
    const int passes = (rows + RPP - 1) / RPP;
    using Full = std::integral_constant<int, RA>;
    using Half = std::integral_constant<int, (RA % 2 == 0 ? RA / 2 : RA)>;
    using Quarter = std::integral_constant<int, (RA % 4 == 0 ? RA / 4 : RA)>;
    using Two = std::integral_constant<int, 2>;
    // Only the bf16 128-row shapes take the shorter paths: in fp8 three
    // copies of the body do not fit the register budget together, and the
    // 64-row gate/up shape spills more and ran slower with them.
    constexpr bool kPaths = !C::FP8 && BM == 128;
    if (kPaths && RA % 4 == 0 && passes <= RA / 4)
      body(Quarter{}, Two{});
    else if (kPaths && RA % 2 == 0 && passes <= RA / 2)
      body(Half{}, Two{});
    else
      body(Full{}, std::integral_constant<int, AD>{});
    if constexpr (SYNC == kSignal) {
      // every thread's z stores have reached the device-wide point of
      // coherence before the tile counter says so
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      if (tid == 0) __hip_atomic_fetch_add(sync + 1 + ti, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // the next item's first barrier orders these LDS reads before reuse
  }
}

template <Elem EL, int WAVES, int BM, int SS, bool SWIGLU, int AD>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(2))) void stream_gemm_kernel(const GemmArgs p) {
  using C = StreamCfg<EL, WAVES, BM, SS, SWIGLU>;
  __shared__ __align__(16) uint8_t lds[C::LDS];
  // fp8: activation scale x weight block scale, [buffer][matrix][K block][row]
  __shared__ __align__(16) typename C::SAs sAs;
  __shared__ int s_item;
  const int total = *p.num_tiles * ((p.N > p.Ns ? p.N : p.Ns) / C::BN);
  for (;;) {
    __syncthreads();  // every thread has read the previous s_item
    if (threadIdx.x == 0) s_item = atomicAdd(p.work_counter, 1);
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(s_item);
    if (item >= total) break;
    stream_item<EL, WAVES, BM, SS, SWIGLU, AD, kNoSync>(p, item, lds, sAs, nullptr);
  }
}

// Both weight-streaming GEMMs of a bf16 decode forward in one persistent
// launch: the workgroups claim the gate/up items (8 waves x 64 rows x 128 z
// columns) and then the down items (8 waves x 64 rows x 128 output columns,
// or with WIDE two 128-column weight blocks per item, so a row tile's z rows
// are staged half as often per weight byte) from one counter, so the last
// gate/up items run beside the first down items instead of leaving CUs idle
// before a second launch.  A down item starts
// once every gate/up item of its row tile has finished (tile counters,
// zeroed by the dispatch kernel).  Per item the arithmetic is that of the
// separate launches, so the results are bitwise the same.
template <int SSG, int SSD, bool WIDE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2))) void stream_ffn_kernel(
    const GemmArgs gu, const GemmArgs dn, int32_t *sync) {
  using CG = StreamCfg<Elem::BF16, 8, 64, SSG, true>;
  using CD = StreamCfg<Elem::BF16, 8, 64, SSD, false, WIDE>;
  constexpr int kLds = CG::LDS > CD::LDS ? CG::LDS : CD::LDS;
  __shared__ __align__(16) uint8_t lds[kLds];
  __shared__ __align__(16) typename CG::SAs sAsG;
  __shared__ __align__(16) typename CD::SAs sAsD;
  __shared__ int s_item;
  const int n_gu = *gu.num_tiles * ((gu.N > gu.Ns ? gu.N : gu.Ns) / CG::BN);
  const int n_all = n_gu + *dn.num_tiles * ((dn.N > dn.Ns ? dn.N : dn.Ns) / CD::ICOLS);
  for (;;) {
    __syncthreads();  // every thread has read the previous s_item
    if (threadIdx.x == 0) s_item = atomicAdd(gu.work_counter, 1);
    __syncthreads();
    const int item = __builtin_amdgcn_readfirstlane(s_item);
    if (item >= n_all) break;
    if (item < n_gu)
      stream_item<Elem::BF16, 8, 64, SSG, true, 1, kSignal>(gu, item, lds, sAsG, sync);
    else
      stream_item<Elem::BF16, 8, 64, SSD, false, 2, kWait, CG::BN, WIDE>(dn, item - n_gu, lds,
                                                                           sAsD, sync);
  }
}

template <Elem EL, int WAVES, int BM, int SS, bool SWIGLU, int AD = 1>
hipError_t launch_stream(const GemmArgs &a, hipStream_t s) {
  auto kern = stream_gemm_kernel<EL, WAVES, BM, SS, SWIGLU, AD>;
  // resident workgroups of this kernel on the current device (cached per device)
  constexpr int kMaxDevices = 64;
  static std::atomic<int> resident[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  int slots = resident[dev].load(std::memory_order_relaxed);
  if (slots <= 0) {
    int cus = 0, per_cu = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(kern),
                                                     WAVES * 64, 0);
    if (e != hipSuccess || per_cu < 1) per_cu = 1;
    slots = cus * per_cu;
    resident[dev].store(slots, std::memory_order_relaxed);
  }
  constexpr int BN = 16 * WAVES;
  const int nmax = a.N > a.Ns ? a.N : a.Ns;
  const int64_t items = static_cast<int64_t>(a.tiles_ub) * (nmax / BN);
  // persistent: one resident wave of workgroups
  int64_t grid = slots;
  if (items < grid) grid = items;
  if (grid <= 0) return hipSuccess;
  kern<<<static_cast<unsigned>(grid), WAVES * 64, 0, s>>>(a);
  return hipGetLastError();
}

// Down items 256 columns wide when there are few per resident workgroup
// (fewer than this many 128-column items): there each item's start is a
// large share of its time (decode h4096 layer: 0.502 against 0.521 ms per
// forward with 128-column items; DeepSeek-V3 EP8 shard 0.522 against
// 0.537); with many items the narrow ones measured 1% faster (DeepSeek-V3
// decode).  Both widths give the same bits.
constexpr int kWideBelowItemsPerSlot = 32;

template <int SSG, int SSD, bool WIDE>
hipError_t launch_ffn(const GemmArgs &gu, const GemmArgs &dn, int32_t *sync, hipStream_t s,
                      int slots) {
  const int64_t items =
      static_cast<int64_t>(gu.tiles_ub) * ((gu.N > gu.Ns ? gu.N : gu.Ns) / 128 +
                                           (dn.N > dn.Ns ? dn.N : dn.Ns) / (WIDE ? 256 : 128));
  int64_t grid = slots;
  if (items < grid) grid = items;
  if (grid <= 0) return hipSuccess;
  stream_ffn_kernel<SSG, SSD, WIDE><<<static_cast<unsigned>(grid), 512, 0, s>>>(gu, dn, sync);
  return hipGetLastError();
}

// resident workgroups of the single launch on the current device (every
// instantiation has the same block size and holds one workgroup per CU)
hipError_t ffn_slots(int *slots_out) {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> resident[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  int slots = resident[dev].load(std::memory_order_relaxed);
  if (slots <= 0) {
    int cus = 0, per_cu = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per_cu, reinterpret_cast<const void *>(stream_ffn_kernel<512, 512, true>), 512, 0);
    if (e != hipSuccess || per_cu < 1) per_cu = 1;
    slots = cus * per_cu;
    resident[dev].store(slots, std::memory_order_relaxed);
  }
  *slots_out = slots;
  return hipSuccess;
}

}  // namespace

bool stream_gate_up_writes_fp8(int elem, int bm) { return elem == 2 && bm == 128; }

bool stream_ffn_supported(int elem, int bm, int hidden, int inter, int shared_inter) {
  // gate/up items of 128 z columns (I, I_s multiples of 128) and down items
  // of 256 output columns; gate/up stages 512 bytes of K
  return elem == 1 && bm == 64 && hidden % 256 == 0 && inter % 128 == 0 &&
         shared_inter % 128 == 0;
}

hipError_t launch_ffn_stream(const GemmArgs &gu, const GemmArgs &dn, int32_t *sync,
                             hipStream_t s) {
  if (!stream_ffn_supported(1, 64, gu.K, gu.N, gu.Ns) || gu.K != gu.Ks || dn.N != gu.K ||
      dn.K != gu.N || dn.Ks != gu.Ns || gu.tiles != dn.tiles || gu.num_tiles != dn.num_tiles)
    return hipErrorInvalidValue;
  int slots = 0;
  hipError_t e = ffn_slots(&slots);
  if (e != hipSuccess) return e;
  const int64_t narrow = static_cast<int64_t>(gu.tiles_ub) * ((dn.N > dn.Ns ? dn.N : dn.Ns) / 128);
  const bool wide = narrow < static_cast<int64_t>(kWideBelowItemsPerSlot) * slots;
  // down: 512-byte stages where every K allows them
  const bool ss512 = dn.K % 256 == 0 && dn.Ks % 256 == 0;
  if (wide)
    return ss512 ? launch_ffn<512, 512, true>(gu, dn, sync, s, slots)
                 : launch_ffn<512, 256, true>(gu, dn, sync, s, slots);
  return ss512 ? launch_ffn<512, 512, false>(gu, dn, sync, s, slots)
               : launch_ffn<512, 256, false>(gu, dn, sync, s, slots);
}

hipError_t launch_gemm_stream(GemmKind kind, int elem, int bm, const GemmArgs &a,
                              hipStream_t s) {
  const bool gu = kind == GemmKind::GateUp;
  const int64_t es = elem == 2 ? 1 : 2;
  // every group's K (bytes per row) must be whole super-stages
  auto fits = [&](int64_t ss) { return (a.K * es) % ss == 0 && (a.Ks * es) % ss == 0; };
  if (elem == 1) {
    if (bm == 64) {
      if (gu) {
        // With many items per resident workgroup (DeepSeek-V3 decode shapes)
        // 8 waves x 128 columns stage each activation row half as often; with
        // few (3 per workgroup on the decode h4096 layer) the 4-wave shape's
        // smaller items finish closer together.
        const int nmax = a.N > a.Ns ? a.N : a.Ns;
        const int64_t items128 = static_cast<int64_t>(a.tiles_ub) * (nmax / 128);
        if (fits(512) && items128 >= 2048)
          return launch_stream<Elem::BF16, 8, 64, 512, true>(a, s);
        return fits(512) ? launch_stream<Elem::BF16, 4, 64, 512, true>(a, s)
                         : launch_stream<Elem::BF16, 4, 64, 128, true>(a, s);
      }
      return fits(512) ? launch_stream<Elem::BF16, 8, 64, 512, false, 2>(a, s)
                       : launch_stream<Elem::BF16, 8, 64, 256, false, 2>(a, s);
    }
    if (bm == 128) {
      if (gu)
        return fits(256) ? launch_stream<Elem::BF16, 4, 128, 256, true>(a, s)
                         : launch_stream<Elem::BF16, 4, 128, 128, true>(a, s);
      return fits(256) ? launch_stream<Elem::BF16, 8, 128, 256, false, 2>(a, s)
                       : launch_stream<Elem::BF16, 8, 128, 128, false>(a, s);
    }
  } else if (elem == 2) {
    if (bm == 64) {
      if (gu)
        return fits(256) ? launch_stream<Elem::FP8, 4, 64, 256, true>(a, s)
                         : launch_stream<Elem::FP8, 4, 64, 128, true>(a, s);
      return launch_stream<Elem::FP8, 4, 64, 128, false>(a, s);
    }
    if (bm == 128)
      // both gate/up shapes are 128 columns wide: stream_gate_up_writes_fp8
      return gu ? (fits(256) ? launch_stream<Elem::FP8, 8, 128, 256, true, 2>(a, s)
                          : launch_stream<Elem::FP8, 8, 128, 128, true>(a, s))
                : launch_stream<Elem::FP8, 8, 128, 128, false, 2>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace afd
