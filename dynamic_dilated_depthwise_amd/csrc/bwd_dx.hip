// bwd_dx.hip -- dX of the fused training backward, tap recompute + gather (gfx950).
//
// Operation (page "lartpang/DynamicConvolutionOperator", section
// "CUDA Flash 式融合训练": the backward recomputes the taps instead of storing
// them):
//     dX[c, q] = G_x[c, q] + sum_{b,t} T[o(b,c,t), q - d_bt] * G_b[c, q - d_bt],
//     T[o, p]  = bias[o] + sum_c' W[o, c'] y[c', p].
// For every (b, t) the generator block is run on y at the shifted pixels q - d_bt,
// so the lane that owns output pixel q receives the tap applied at its source
// pixel; it is multiplied by G_b at that same pixel (zero outside the image, which
// also removes the bias-only taps recomputed there).  A gather: every dX element
// is stored once, no atomics, no halo recompute.
//
// Workgroup = one 64-pixel row segment x 64 output channels; wave v owns the
// 16-channel block 16v (MFMA rows = 16 channels of one (b, t) pair, columns = 16
// lanes x 4 adjacent pixels, as in the fused forward).  All four waves need the
// same B operand -- y at the shifted segment, every input channel -- so it is
// staged once per (tap, 64-channel chunk) in LDS, double-buffered: the next
// stage's y, weight fragments and G_b are loaded while the current stage's MFMAs
// run, with one barrier per stage.
//   float32: LDS rows [channel][pixel], padded to 68 floats so that the staging
//     writes and the 16-byte fragment reads are free of bank conflicts;
//   bfloat16: LDS rows [pixel][channel] (the MFMA operand is 8 consecutive
//     channels of one pixel), 16-byte channel chunks XOR-swizzled by pixel/4 so
//     the lanes of a fragment read hit distinct banks.
#include "gen_mma.hpp"
#include "launchers.hpp"

namespace ddpm {
namespace {

constexpr int kSeg = 64;    // pixels per row segment (16 lanes x 4)
constexpr int kChunk = 64;  // input channels per stage
constexpr int kOutCh = 64;  // output channels per workgroup (16 per wave)
constexpr int kCUs = 256;   // compute units of the chip (MI355X)

template <typename T> struct DxStage;

template <> struct DxStage<float> {
    static constexpr int ROW = kSeg + 4;      // floats per staged channel row
    static constexpr int ELEMS = kChunk * ROW;
    static constexpr int SUB = 4;             // 16-channel MFMA chunks per stage
    struct Regs { f32x4 v[4]; };

    // Thread tid (0..255 within its wave group) stages channel tid/4 of the chunk,
    // pixels 16*(tid%4) .. +15 of the shifted segment starting at column ws0.
    __device__ __forceinline__ static void load(Regs &R, int tid, const float *__restrict__ yn, int c_first, int C,
                                                int64_t HW, int64_t rowoff, int ws0, int W, bool row_ok,
                                                bool fast, bool al) {
        const int c = c_first + (tid >> 2);
        const int px = ws0 + 16 * (tid & 3);
        const float *row = yn + (int64_t)(c < C ? c : 0) * HW + rowoff;
        const bool al4 = al && ((px & 3) == 0);  // 16-byte aligned runs (rows are, when al)
        if (fast) {
#pragma unroll
            for (int i = 0; i < 4; ++i) R.v[i] = load4_unchecked(row, px + 4 * i, al4, true, false);
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) R.v[i] = load4_row(row, px + 4 * i, W, row_ok && c < C, al4);
        }
    }
    __device__ __forceinline__ static void store(float *__restrict__ buf, int tid, const Regs &R) {
        float *p = buf + (tid >> 2) * ROW + 16 * (tid & 3);
#pragma unroll
        for (int i = 0; i < 4; ++i) *(f32x4 *)(p + 4 * i) = R.v[i];
    }
    // B fragment of MFMA chunk `sub`: v[s][pb] = y[16 sub + 4g + s][4j + pb].
    __device__ __forceinline__ static Gen<float>::BFrag frag(const float *__restrict__ buf, int sub, int g, int j) {
        Gen<float>::BFrag b;
#pragma unroll
        for (int s = 0; s < 4; ++s) b.v[s] = *(const f32x4 *)(buf + (16 * sub + 4 * g + s) * ROW + 4 * j);
        return b;
    }
};

template <> struct DxStage<bf16_t> {
    static constexpr int ELEMS = kSeg * kChunk;  // [pixel][64 channels], 128-byte rows
    static constexpr int SUB = 2;                // 32-channel MFMA chunks per stage
    struct Regs { u16x4 v[4]; };                 // v[channel i][pixel p]

    __device__ __forceinline__ static int slot(int P, int chunk) { return P * kChunk + 8 * (chunk ^ ((P >> 2) & 7)); }

    // Raw bits of row[px .. px+3].  fast: in range (px >= 1 when odd); al4: 8-byte
    // aligned run; row4: the row start is 4-byte aligned.  Otherwise zero outside
    // [0, W) or when !ok.
    __device__ __forceinline__ static u16x4 run4(const bf16_t *__restrict__ row, int px, int W, bool ok, bool fast,
                                                 bool al4, bool row4, bool odd) {
        if (fast) {
            if (al4) return *(const u16x4 *)(row + px);
            if (row4 && !odd) return __builtin_bit_cast(u16x4, *(const u32x2_a4 *)(row + px));
            if (row4) {
                const u32x2_a4 d = *(const u32x2_a4 *)(row + px - 1);
                u16x4 u;
                u[0] = (uint16_t)(d[0] >> 16); u[1] = (uint16_t)d[1]; u[2] = (uint16_t)(d[1] >> 16);
                u[3] = row[px + 3];
                return u;
            }
        }
        u16x4 u = {0, 0, 0, 0};
        if (!ok) return u;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int ww = px + k;
            if (fast || (ww >= 0 && ww < W)) u[k] = row[ww];
        }
        return u;
    }

    // Thread tid (0..255 within its wave group) stages channels 4*(tid/16) .. +3 of
    // the chunk, pixels 4*(tid%16) .. +3.
    __device__ __forceinline__ static void load(Regs &R, int tid, const bf16_t *__restrict__ yn, int c_first, int C,
                                                int64_t HW, int64_t rowoff, int ws0, int W, bool row_ok,
                                                bool fast, bool al) {
        const int px = ws0 + 4 * (tid & 15);
        const bool odd = (ws0 & 1) != 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = c_first + 4 * (tid >> 4) + i;
            const bf16_t *row = yn + (int64_t)(c < C ? c : 0) * HW + rowoff;
            R.v[i] = run4(row, px, W, row_ok && c < C, fast, al && ((px & 3) == 0), al, odd);
        }
    }
    __device__ __forceinline__ static void store(bf16_t *__restrict__ buf, int tid, const Regs &R) {
        const int c4 = 4 * (tid >> 4);
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int P = 4 * (tid & 15) + p;
            u16x4 u;
            u[0] = R.v[0][p]; u[1] = R.v[1][p]; u[2] = R.v[2][p]; u[3] = R.v[3][p];
            *(u16x4 *)(buf + slot(P, c4 >> 3) + (c4 & 4)) = u;
        }
    }
    // B fragment of MFMA chunk `sub`: v[pb] = y[32 sub + 8g + e][4j + pb], e = 0..7.
    __device__ __forceinline__ static Gen<bf16_t>::BFrag frag(const bf16_t *__restrict__ buf, int sub, int g,
                                                              int j) {
        Gen<bf16_t>::BFrag b;
#pragma unroll
        for (int pb = 0; pb < 4; ++pb)
            b.v[pb] = __builtin_bit_cast(bf16x8, *(const u16x8 *)(buf + slot(4 * j + pb, 4 * sub + g)));
        return b;
    }
};

// NG = 1: four waves, one per 16-channel block, run every stage.  NG = 2 or 4 (small
// grids): NG groups of four waves, each with its own staging buffers, take
// consecutive whole-tap shares of the stages in lockstep (the shared barriers), and
// the other groups' sums are added to the first's in group order at the end -- NG
// times the waves per SIMD for the same tile.
template <typename T, int K, int NG, bool FULLW>
__global__ __launch_bounds__(256 * NG, NG == 4 ? 4 : (NG == 1 ? 2 : 1)) void bwd_dx_kernel(const T *__restrict__ y,
                                                                          const T *__restrict__ wg,
                                                                          const T *__restrict__ bg,
                                                                          const T *__restrict__ gout,
                                                                          T *__restrict__ gx, int C, int H, int W,
                                                                          int al) {
    using G = Gen<T>;
    using S = DxStage<T>;
    constexpr int r = (K - 1) / 2;
    constexpr int KK = K * K;
    const int lane = threadIdx.x & 63;
    const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int grp = NG == 1 ? 0 : wave_all >> 2;                      // wave group
    const int wave = NG == 1 ? wave_all : wave_all & 3;                // 16-channel block within it
    const int tid = NG == 1 ? (int)threadIdx.x : (int)threadIdx.x & 255;  // thread within the group
    const int g = lane >> 4;
    const int j = lane & 15;
    // logical tile order: channel group fastest, then column segment, row, image
    const int ncg = (C + kOutCh - 1) / kOutCh;
    const int nseg = (W + kSeg - 1) / kSeg;
    int L = xcd_contiguous(blockIdx.x, gridDim.x);
    const int cg0 = (L % ncg) * kOutCh;
    L /= ncg;
    const int w0 = (L % nseg) * kSeg;
    L /= nseg;
    const int h = L % H;
    const int n = L / H;
    const int c0 = cg0 + 16 * wave;             // this wave's output channel block
    const bool wave_on = c0 < C;                // wave-uniform
    const int w = w0 + 4 * j;
    const int cA = c0 + j;                      // generator row channel this lane supplies
    const int64_t HW = (int64_t)H * W;
    const bool aligned4 = al != 0;
    const bool cvec = Elem<T>::is_bf16 ? (al != 0 && (C & 7) == 0) : (al != 0 && (C & 3) == 0);
    // All 16 channels of the block exist, weights are vector-aligned, and 32-bit lane
    // offsets address a 16-plane G slice (wave-uniform).
    const bool full = (c0 + 16 <= C) && cvec && HW < (int64_t(1) << 26);
    const int HWi = (int)(full ? HW : 0);
    const T *__restrict__ yn = y + (int64_t)n * C * HW;
    const T *__restrict__ gn = gout + (int64_t)n * 4 * C * HW;
    const int nqq = (C + kChunk - 1) / kChunk;
    const int nstage = 3 * KK * nqq;
    // this group's stages [sb, se), whole taps (all nqq chunks of a tap stay in one
    // group); every group runs `nit` lockstep iterations
    const int cpg = (3 * KK + NG - 1) / NG;  // taps per group
    const int nit = cpg * nqq;
    const int sb = grp * nit;
    const int se = min(nstage, sb + nit);

    // float32 keeps few registers live (weight fragments one MFMA chunk ahead, G_b
    // loaded at the start of the stage that uses it: a stage holds 2048 MFMA cycles),
    // so four workgroups fit a CU; bfloat16 stages are short, so everything a stage
    // needs is fetched one whole stage ahead.
    constexpr bool AHEAD = Elem<T>::is_bf16;
    __shared__ __align__(16) T stage[NG][2][S::ELEMS];
    // bfloat16: the biases of this workgroup's channels for every tap, staged once
    // (bl[(b*KK + t)*64 + ch]); float32 loads a tap's biases with its G_b.
    __shared__ float bl[AHEAD ? 3 * KK * kOutCh : 1];
    if constexpr (AHEAD) {
        for (int i = threadIdx.x; i < 3 * KK * kOutCh; i += blockDim.x) {
            const int combo = i / kOutCh;
            const int c = cg0 + (i - combo * kOutCh);
            const int b = combo / KK;
            const int t = combo - b * KK;
            bl[i] = c < C ? Elem<T>::to_f32(bg[(int64_t)(b * C + c) * KK + t]) : 0.f;
        }
    }

    struct Shift {
        int b, t, hs, dc;
        bool row_ok;
    };
    // Stages are (combo = b*KK + t, chunk qq), qq fastest; the loop carries both so
    // no division by the run-time chunk count is needed (K is a constant).
    auto shift_of = [&](int combo) {
        Shift sh;
        sh.b = combo / KK;
        sh.t = combo - sh.b * KK;
        const int D = dilation(sh.b);
        const int ki = sh.t / K;
        const int kj = sh.t - ki * K;
        sh.hs = h - (ki - r) * D;
        sh.dc = (kj - r) * D;
        sh.row_ok = sh.hs >= 0 && sh.hs < H;
        return sh;
    };
    // y of stage (combo, qq) (shifted segment, one 64-channel chunk) into staging registers
    auto load_stage = [&](int combo, int qq, typename S::Regs &R) {
        const Shift sh = shift_of(combo);
        const int ws0 = w0 - sh.dc;
        const int64_t rowoff = (int64_t)(sh.row_ok ? sh.hs : 0) * W;
        const bool fast = (kChunk * qq + kChunk <= C) && sh.row_ok && ws0 - (ws0 & 1) >= 0 && ws0 + kSeg <= W;
        S::load(R, tid, yn, kChunk * qq, C, HW, rowoff, ws0, W, sh.row_ok, fast, aligned4);
    };
    // weight fragment of MFMA chunk u of stage (combo, qq) for this wave's 16 generator rows
    auto load_A1 = [&](int combo, int qq, int u, typename G::AFrag &a) {
        const int b = combo / KK;
        const int t = combo - b * KK;
        const int q = S::SUB * qq + u;  // MFMA chunk of G::CH input channels
        if (FULLW || (full && kChunk * qq + kChunk <= C)) {
            a = G::load_A_off(wg + ((int64_t)b * C * KK + t) * C, cA * KK * C + G::CH * q + (G::CH / 4) * g);
        } else {
            const T *arow = cA < C ? wg + ((int64_t)(b * C + cA) * KK + t) * C : nullptr;
            a = G::load_A(arow, q, g, C, cvec);
        }
    };
    // all weight fragments of stage (combo, qq)
    auto load_A = [&](int combo, int qq, typename G::AFrag (&a)[S::SUB]) {
        const Shift sh = shift_of(combo);
#pragma unroll
        for (int u = 0; u < S::SUB; ++u) {
            const int q = S::SUB * qq + u;
            if (full && kChunk * qq + kChunk <= C) {
                a[u] = G::load_A_off(wg + ((int64_t)sh.b * C * KK + sh.t) * C, cA * KK * C + G::CH * q +
                                                                                    (G::CH / 4) * g);
            } else {
                const T *arow = cA < C ? wg + ((int64_t)(sh.b * C + cA) * KK + sh.t) * C : nullptr;
                a[u] = G::load_A(arow, q, g, C, cvec);
            }
        }
    };
    // generator bias of tap `combo` for channels c0+4g+v
    auto load_bias = [&](int combo, f32x4 &bv) {
        const int b = combo / KK;
        const int t = combo - b * KK;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int c = c0 + 4 * g + v;
            bv[v] = c < C ? Elem<T>::to_f32(bg[(int64_t)(b * C + c) * KK + t]) : 0.f;
        }
    };
    // G_b at the source pixels of tap `combo`: gs[v][pb] for channel c0+4g+v
    auto load_G = [&](int combo, f32x4 (&gs)[4]) {
        const Shift sh = shift_of(combo);
        const int ws = w - sh.dc;
        const int odd = sh.dc & 1;
        const bool al_s = aligned4 && ((sh.dc & 3) == 0);
        const int64_t rowoff = (int64_t)(sh.row_ok ? sh.hs : 0) * W;
        if (full && sh.row_ok && w0 - sh.dc - odd >= 0 && w0 + kSeg - 1 - sh.dc < W) {  // wave-uniform
            const T *gbase = gn + (int64_t)((1 + sh.b) * C + c0) * HW + rowoff;
            const int goff = 4 * g * HWi + ws;
#pragma unroll
            for (int v = 0; v < 4; ++v) gs[v] = load4_unchecked(gbase + (int64_t)v * HWi, goff, al_s, aligned4, odd);
        } else {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int c = c0 + 4 * g + v;
                gs[v] = load4_row(gn + (int64_t)((1 + sh.b) * C + (c < C ? c : 0)) * HW + rowoff, ws, W,
                                  sh.row_ok && c < C, al_s);
            }
        }
    };

    const bool grp_on = NG == 1 || sb < se;  // wave-uniform: the group has stages
    int combo = sb / nqq, qq = sb - (sb / nqq) * nqq;  // current stage
    typename S::Regs R;
    if (grp_on) {
        load_stage(combo, qq, R);
        S::store(stage[grp][0], tid, R);
    }
    typename G::AFrag acur[AHEAD ? S::SUB : 1];
    f32x4 gcur[4], gnext[4], bcur = f32x4{0.f, 0.f, 0.f, 0.f};
    if (wave_on && grp_on) {
        if constexpr (AHEAD) {
            load_A(combo, qq, acur);
            load_G(combo, gcur);
        } else {
            load_A1(combo, qq, 0, acur[0]);
        }
    }
    float dacc[4][4];
#pragma unroll
    for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) dacc[v][pb] = 0.f;
    f32x4 acc[4];
    __syncthreads();

#pragma unroll 1
    for (int it = 0; it < nit; ++it) {
        const int s = sb + it;
        const bool act = NG == 1 || s < se;  // wave-uniform: this group has a stage this round
        const bool more = s + 1 < se;
        const int qn = qq + 1 == nqq ? 0 : qq + 1;  // next stage
        const int cn = qn == 0 ? combo + 1 : combo;
        typename G::AFrag anext[S::SUB];  // bfloat16: the next stage's fragments
        if (more) {
            load_stage(cn, qn, R);
            if constexpr (AHEAD) {
                if (wave_on) {
                    load_A(cn, qn, anext);
                    if (qn == 0) load_G(cn, gnext);
                }
            }
        }
        if (wave_on && act) {
            const bool last = qq == nqq - 1;  // the tap's last chunk: its G_b term follows
            const T *buf = stage[grp][it & 1];
            const int left = C - kChunk * qq;
            const int nsub = left >= kChunk ? S::SUB : (left + G::CH - 1) / G::CH;
            if (qq == 0) {
                // bfloat16: the sum starts at the bias; float32 adds it at the end
                const f32x4 a0 = AHEAD ? *(const f32x4 *)(bl + combo * kOutCh + 16 * wave + 4 * g)
                                       : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int pb = 0; pb < 4; ++pb) acc[pb] = a0;
            }
            if constexpr (AHEAD) {
#pragma unroll
                for (int u = 0; u < S::SUB; ++u)
                    if (u < nsub) G::mma(acc, acur[u], S::frag(buf, u, g, j));
                if (more) {
#pragma unroll
                    for (int u = 0; u < S::SUB; ++u) acur[u] = anext[u];
                }
            } else {
                if (last) {
                    load_G(combo, gcur);
                    load_bias(combo, bcur);
                }
                // one wave group: raised issue priority while the stage's MFMAs go out
                // (with two or four lockstep groups it measured slower)
                if constexpr (NG == 1) __builtin_amdgcn_s_setprio(1);
#pragma unroll
                for (int u = 0; u < S::SUB; ++u) {
                    if (FULLW) {
                        // Whole chunks, aligned weights: the next fragment (this one again
                        // after the last) is one load on every path, so the wait before the
                        // MFMAs can leave it in flight (with loads on some paths only, the
                        // compiler has to wait for all of them there).
                        typename G::AFrag an;
                        const bool in_stage = u + 1 < S::SUB;
                        load_A1(in_stage ? combo : (more ? cn : combo), in_stage ? qq : (more ? qn : qq),
                                in_stage ? u + 1 : (more ? 0 : u), an);
                        G::mma(acc, acur[0], S::frag(buf, u, g, j));
                        acur[0] = an;
                    } else if (u < nsub) {
                        typename G::AFrag an;
                        const bool in_stage = u + 1 < nsub;
                        if (in_stage) load_A1(combo, qq, u + 1, an);
                        else if (more) load_A1(cn, qn, 0, an);
                        G::mma(acc, acur[0], S::frag(buf, u, g, j));
                        if (in_stage || more) acur[0] = an;
                    }
                }
                if constexpr (NG == 1) __builtin_amdgcn_s_setprio(0);
            }
            if (last) {
                // the bias is in the fp32 sum before the tap's single rounding
#pragma unroll
                for (int v = 0; v < 4; ++v)
#pragma unroll
                    for (int pb = 0; pb < 4; ++pb) {
                        const float tap = AHEAD ? acc[pb][v] : acc[pb][v] + bcur[v];
                        dacc[v][pb] += Elem<T>::quant(tap) * gcur[v][pb];
                    }
                if (AHEAD && more) {
#pragma unroll
                    for (int v = 0; v < 4; ++v) gcur[v] = gnext[v];
                }
            }
        }
        if (more) S::store(stage[grp][(it + 1) & 1], tid, R);
        __syncthreads();
        combo = cn;
        qq = qn;
    }

    if constexpr (NG > 1) {
        // the other groups' sums, each through its own (now idle) staging buffers,
        // added to the first group's in group order: dX = G_x + ((taps of group 0 +
        // taps of group 1) + ...).  The buffers are reused as float storage (16 KB,
        // within both dtypes' 2 * ELEMS); the barriers before the stores and before
        // the loads order every access.
        if (grp > 0 && wave_on) {
            float *xfer = reinterpret_cast<float *>(&stage[grp][0][0]);
#pragma unroll
            for (int v = 0; v < 4; ++v)
                *(f32x4 *)(xfer + ((wave * 64 + lane) * 4 + v) * 4) =
                    f32x4{dacc[v][0], dacc[v][1], dacc[v][2], dacc[v][3]};
        }
        __syncthreads();
        if (grp > 0) return;
        if (wave_on) {
#pragma unroll
            for (int k = 1; k < NG; ++k) {
                const float *xfer = reinterpret_cast<const float *>(&stage[k][0][0]);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const f32x4 o = *(const f32x4 *)(xfer + ((wave * 64 + lane) * 4 + v) * 4);
#pragma unroll
                    for (int pb = 0; pb < 4; ++pb) dacc[v][pb] += o[pb];
                }
            }
        }
    }
    if (!wave_on) return;
    const int64_t rowoff = (int64_t)h * W;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int c = c0 + 4 * g + v;
        if (c >= C || w >= W) continue;
        const f32x4 gxs = load4_row(gn + (int64_t)c * HW + rowoff, w, W, true, aligned4);
        f32x4 o;
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) o[pb] = dacc[v][pb] + gxs[pb];
        store4_row(gx + ((int64_t)n * C + c) * HW + rowoff, w, W, o, aligned4);
    }
}

template <typename T, int K>
hipError_t launch_dx_t(const void *y, const void *wg, const void *bg, const void *gout, void *gx, int N, int C, int H,
                       int W, bool al, hipStream_t stream) {
    const int64_t nblk = bwd_dx_blocks(N, C, H, W);
    if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    // more wave groups per workgroup on small grids: four when the grid gives at most
    // one workgroup per CU, two when at most two
    // float32 with whole 64-channel chunks and aligned rows: single-path weight prefetch
    const bool fullw = !Elem<T>::is_bf16 && al && C % kChunk == 0 && (int64_t)H * W < (int64_t(1) << 26);
    auto launch = [&](auto kern, int threads) {
        hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(threads), 0, stream, (const T *)y, (const T *)wg,
                           (const T *)bg, (const T *)gout, (T *)gx, C, H, W, al ? 1 : 0);
    };
    // row-staged kernel from one 64-pixel segment per CU up (measured at 128x128,
    // C = 64: K = 5 bf16 140 -> 55 us, fp32 146 -> 108 us; K = 3 bf16 60 -> 28 us)
    if (nblk >= kCUs && bwd_dx_rows_applies(C, H, W, al, Elem<T>::is_bf16))
        return launch_bwd_dx_rows(y, wg, bg, gout, gx, N, H, W, K, Elem<T>::is_bf16, stream);
    if (nblk <= kCUs) {
        if (fullw) launch(bwd_dx_kernel<T, K, 4, !Elem<T>::is_bf16>, 1024);
        else launch(bwd_dx_kernel<T, K, 4, false>, 1024);
    } else if (nblk <= 2 * kCUs) {
        if (fullw) launch(bwd_dx_kernel<T, K, 2, !Elem<T>::is_bf16>, 512);
        else launch(bwd_dx_kernel<T, K, 2, false>, 512);
    } else {
        if (fullw) launch(bwd_dx_kernel<T, K, 1, !Elem<T>::is_bf16>, 256);
        else launch(bwd_dx_kernel<T, K, 1, false>, 256);
    }
    return hipGetLastError();
}

}  // namespace

int64_t bwd_dx_blocks(int N, int C, int H, int W) {
    return (int64_t)N * H * ((W + kSeg - 1) / kSeg) * ((C + kOutCh - 1) / kOutCh);
}

hipError_t launch_bwd_dx(const void *y, const void *wg, const void *bg, const void *gout, void *gx, int N, int C,
                         int H, int W, int K, bool bf16, bool al, hipStream_t stream) {
    if (bf16) {
        switch (K) {
            case 1: return launch_dx_t<bf16_t, 1>(y, wg, bg, gout, gx, N, C, H, W, al, stream);
            case 3: return launch_dx_t<bf16_t, 3>(y, wg, bg, gout, gx, N, C, H, W, al, stream);
            default: return launch_dx_t<bf16_t, 5>(y, wg, bg, gout, gx, N, C, H, W, al, stream);
        }
    }
    switch (K) {
        case 1: return launch_dx_t<float, 1>(y, wg, bg, gout, gx, N, C, H, W, al, stream);
        case 3: return launch_dx_t<float, 3>(y, wg, bg, gout, gx, N, C, H, W, al, stream);
        default: return launch_dx_t<float, 5>(y, wg, bg, gout, gx, N, C, H, W, al, stream);
    }
}

}  // namespace ddpm
