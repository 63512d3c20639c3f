// Host check of libfs's launch planning and workspace layout (fs_plan.cpp),
// built on the CPU with address and undefined-behaviour sanitizers by
// tests/test_plan_host.py.  For a grid of shapes, extreme ones included, it
// plans every variant on several compute-unit counts and checks the plan's
// invariants and the layout's bounds, alignment and disjointness.  Prints
// "plan <name> ..." lines for named shapes and "ok <cases>" at the end; any
// violated invariant prints "FAIL ..." and exits with status 1.
#include <algorithm>
#include <climits>
#include <cstdio>
#include <cstdlib>
#include <utility>
#include <vector>

#include "fs_plan.h"

using namespace fs;

namespace {

int g_fail = 0;
long g_cases = 0;
long g_unlaunchable = 0;

#define CHECK(cond, ...)                                             \
    do {                                                             \
        if (!(cond)) {                                               \
            std::printf("FAIL %s:%d %s | ", __FILE__, __LINE__, #cond); \
            std::printf(__VA_ARGS__);                                \
            std::printf("\n");                                       \
            ++g_fail;                                                \
        }                                                            \
    } while (0)

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Every array of the layout: 256-byte aligned, inside the total, disjoint.
void check_layout(const WsLayout& l, const std::vector<std::pair<size_t, size_t>>& arrays,
                  const char* what) {
    std::vector<std::pair<size_t, size_t>> a;
    for (auto& x : arrays)
        if (x.first != kAbsent) a.push_back(x);
    std::sort(a.begin(), a.end());
    size_t end = 0;
    for (auto& x : a) {
        CHECK(x.first % kAlign == 0, "%s offset %zu", what, x.first);
        CHECK(x.first >= end, "%s overlap at %zu", what, x.first);
        CHECK(x.first + x.second <= l.total, "%s array [%zu, +%zu) past total %zu", what, x.first,
              x.second, l.total);
        CHECK(x.second <= l.total, "%s size", what);
        end = x.first + x.second;
    }
}

void check_case(int B, int d, int V, int v_offset, int tile_v, int cus, const char* name) {
    fs_params p{};
    p.B = B;
    p.d = d;
    p.V = V;
    p.v_offset = v_offset;
    p.n_valid = (int)std::min<int64_t>(INT32_MAX, (int64_t)v_offset + V);
    p.tile_v = tile_v;
    p.seed = 0x123456789abcdefull;
    if (check_params(&p) != FS_OK || B == 0 || V == 0) return;
    const int variants[] = {kVarFlat, kVarGrouped, kVarLogits, kVarTopk};
    const int ks[] = {1, 40, 64, 65, 1000, 1024};
    for (int var : variants) {
        Plan pl;
        make_plan(&p, var, cus, pl);
        ++g_cases;
        const int tv = tile_v ? tile_v : kDefaultTileV;
        CHECK(pl.T == cdiv(V, tv), "T");
        CHECK(pl.nmb == cdiv(V, kMBlock), "nmb");
        CHECK(pl.G >= 1 && pl.grid_y >= 1, "G %d grid_y %d", pl.G, pl.grid_y);
        if (!pl.launchable) {   // reported as FS_ERR_UNSUPPORTED: nothing else is used
            ++g_unlaunchable;
            continue;
        }
        CHECK((int64_t)pl.G * pl.grid_y <= kMaxGridX * kMaxGridY, "grid %d x %d", pl.G,
              pl.grid_y);
        CHECK(pl.xcd_pair ? (int64_t)pl.G * pl.grid_y <= kMaxGridX
                          : pl.G <= kMaxGridX && pl.grid_y <= kMaxGridY,
              "grid %d x %d", pl.G, pl.grid_y);
        CHECK(pl.kind >= kCoop && pl.kind <= kRows, "kind %d", pl.kind);
        CHECK(pl.stream == (pl.kind == kStream), "stream flag");
        const int cols = (pl.kind == kWide || pl.kind == kRows) ? pl.nt
                         : pl.kind == kResident                  ? 16 * pl.rcfg.nb
                                                                 : 16 * pl.cfg.nb;
        CHECK(cols >= 16 && (int64_t)pl.grid_y * cols >= B && (int64_t)(pl.grid_y - 1) * cols < B,
              "grid_y %d cols %d B %d", pl.grid_y, cols, B);
        if (pl.kind == kResident) {
            CHECK(pl.rcfg.nw > 0 && resident_supported(pl.rcfg, var), "resident shape");
            CHECK(pl.rcfg.nw * (pl.rcfg.hk + pl.rcfg.hl) == cdiv(d, 32), "resident k-steps");
        }
        if (pl.kind == kRows) {
            CHECK(var == kVarFlat || var == kVarLogits || var == kVarGrouped, "rows variant");
            CHECK(var != kVarGrouped || pl.nt <= 128, "rows grouped columns");
            CHECK(d % (64 * rows_kcs(pl.nt)) == 0, "rows d %d nt %d", d, pl.nt);
        }
        if (pl.kind == kWide || pl.kind == kRows)
            CHECK(pl.nt == 64 || pl.nt == 128 || pl.nt == 256, "nt %d", pl.nt);
        if (pl.kind == kWide) CHECK(var == kVarGrouped && pl.nt == 64, "wide: grouped, 64 columns");
        if (pl.kind == kWide) {   // 32-bit element offsets (the rows kernel forms 64-bit ones)
            CHECK((int64_t)B * d < INT32_MAX, "wide H offsets B %d d %d", B, d);
            CHECK((cdiv(pl.nmb, pl.G) * kMBlock + 256) * d < INT32_MAX, "wide W offsets");
            CHECK(var != kVarGrouped || pl.nt == 64, "wide grouped nt");
        }
        if (pl.kind == kStream) CHECK(pl.G <= std::max(1, pl.nmb / 4), "stream G");
        CHECK(pl.unit_rec == (var == kVarGrouped && (pl.kind == kResident || pl.kind == kRows)),
              "block records");
        const bool strided = pl.kind == kResident && (var != kVarGrouped || pl.unit_rec);
        const int64_t nunits = strided ? cdiv(pl.nmb, pl.rcfg.mpi) : pl.nmb;
        CHECK(pl.G <= nunits, "G %d > units %lld", pl.G, (long long)nunits);
        if (pl.xcd_pair) CHECK(pl.G % 8 == 0 && pl.grid_y > 1, "xcd pairing");
        const int workers = pl.kind == kStream ? 4 * pl.G : pl.G;
        CHECK(pl.P == (pl.unit_rec ? pl.nmb : workers + (var == kVarGrouped ? pl.T - 1 : 0)),
              "P %d", pl.P);
        const int dk = dynamic_k0(pl);
        if (dk > 0) {
            CHECK(var == kVarFlat || var == kVarTopk || pl.unit_rec, "tickets");
            CHECK(dk >= 3 && (int64_t)dk * pl.G <= nunits, "dyn_k0 %d G %d units %lld", dk, pl.G,
                  (long long)nunits);
        }
        const size_t b = (size_t)B, P = (size_t)pl.P;
        if (var == kVarFlat || var == kVarGrouped) {
            const int wv = var == kVarFlat ? FS_VARIANT_FLAT : FS_VARIANT_GROUPED;
            const WsLayout l = layout(wv, pl, 0);
            CHECK(l.pm != kAbsent && l.pidx != kAbsent, "records");
            CHECK((var == kVarGrouped) == (l.pL != kAbsent), "log-mass records");
            CHECK(l.sched != kAbsent, "scheduler block");
            CHECK(pl.stream == (l.part != kAbsent), "partial sums");
            CHECK((var == kVarGrouped && pl.unit_rec) == (l.gsel != kAbsent), "sample pairs");
            CHECK(l.sched + kSchedBytes == l.total, "scheduler block last");
            // block records are block-major, B rounded up to 32 columns per block
            CHECK(pl.rec_cols == (pl.unit_rec ? (B + 31) / 32 * 32 : 0), "record columns");
            const size_t rc = var == kVarGrouped && pl.unit_rec ? (size_t)pl.rec_cols : b;
            check_layout(l, {{l.pm, P * rc * 4}, {l.pidx, P * rc * 4}, {l.pL, P * rc * 4},
                             {l.part, pl.stream ? part_bytes(pl) : 0}, {l.gsel, b * 8 * kGselStride},
                             {l.sched, kSchedBytes}},
                         "records");
            // the multinomial baseline plans with the flat variant
            if (var == kVarFlat) {
                const WsLayout m = layout(FS_VARIANT_MULTINOMIAL, pl, 0);
                const size_t nc = (size_t)cdiv(V, kMultinomialChunk);
                check_layout(m, {{m.mm, nc * b * 4}, {m.ms, nc * b * 4}, {m.mkey, nc * b * 8}},
                             "multinomial");
            }
        } else if (var == kVarLogits) {
            const WsLayout l = layout(FS_VARIANT_LOGITS, pl, 0);
            check_layout(l, {{l.part, pl.stream ? part_bytes(pl) : 0}}, "logits");
        } else {
            for (int k : ks) {
                if (pl.kind != kResident && k > kMaxTopKCoop) continue;   // reported, not run
                if (!topk_launchable(pl, k)) {
                    ++g_unlaunchable;
                    continue;
                }
                const int L = topk_len(pl, k);
                CHECK((int64_t)pl.G * L <= INT32_MAX / 4 && B <= kMaxGridY, "top-k grids");
                const bool dense = topk_dense(pl, k);
                CHECK(L >= 1 && L <= k, "topk_len %d k %d", L, k);
                if (pl.kind == kResident) {
                    const int64_t wg_rows = cdiv(cdiv(pl.nmb, pl.rcfg.mpi), pl.G) *
                                            pl.rcfg.mpi * kMBlock;
                    CHECK(wg_rows <= resident_topk_rows(pl.rcfg), "row store %lld > %d",
                          (long long)wg_rows, resident_topk_rows(pl.rcfg));
                }
                const WsLayout l = layout(FS_VARIANT_TOPK, pl, k);
                const size_t n = (size_t)pl.G * b * (size_t)L;
                const size_t sb = stage2_topk_scratch_bytes(pl.G, L, B, k, dense);
                CHECK(dense == (l.cidx == kAbsent), "dense lists carry no ids");
                check_layout(l, {{l.cx, n * 4}, {l.cidx, n * 4}, {l.sel, sb},
                                 {l.sched, kSchedBytes}},
                             "topk");
            }
        }
        if (name) {
            std::printf("plan %s var=%d kind=%d G=%d grid_y=%d P=%d nt=%d xcd=%d rcfg=%d,%d,%d,%d,%d,%d "
                        "dyn_k0=%d unit_rec=%d\n",
                        name, var, pl.kind, pl.G, pl.grid_y, pl.P, pl.nt, pl.xcd_pair, pl.rcfg.nb,
                        pl.rcfg.mpi, pl.rcfg.ks, pl.rcfg.nw, pl.rcfg.hk, pl.rcfg.hl, dk,
                        pl.unit_rec ? 1 : 0);
        }
    }
}

}  // namespace

int main() {
    // parameter validation: invalid requests never reach the planner
    {
        fs_params p{};
        p.B = 1;
        p.d = 64;
        p.V = 100;
        p.n_valid = 100;
        CHECK(check_params(&p) == FS_OK, "valid");
        p.v_offset = INT32_MAX - 50;
        CHECK(check_params(&p) == FS_ERR_INVALID_ARG, "v_offset + V past INT32_MAX");
        p.v_offset = 0;
        p.d = 12;
        CHECK(check_params(&p) == FS_ERR_UNSUPPORTED, "d %% 8");
        p.d = 64;
        p.tile_v = 24;
        CHECK(check_params(&p) == FS_ERR_UNSUPPORTED, "tile_v %% 16");
        p.tile_v = 0;
        p.B = kMaxB + 1;
        CHECK(check_params(&p) == FS_ERR_UNSUPPORTED, "B limit");
        p.B = 1;
        p.flags = 2;
        CHECK(check_params(&p) == FS_ERR_INVALID_ARG, "flags");
        CHECK(check_params(nullptr) == FS_ERR_INVALID_ARG, "null");
    }
    // named shapes: the configured workloads on a 256-CU device
    check_case(32, 4096, 151936, 0, 0, 256, "headline_b32");
    check_case(1, 4096, 151936, 0, 0, 256, "mid_b1");
    check_case(64, 4096, 151936, 0, 128, 256, "mid_b64");
    check_case(128, 4096, 151936, 0, 0, 256, "sweep_b128");
    check_case(256, 4096, 151936, 0, 0, 256, "sweep_b256");
    check_case(32, 2048, 151936, 0, 256, 256, "small_b32");
    check_case(32, 5120, 152064, 0, 256, 256, "topk_b32");
    check_case(4, 256, 4096, 0, 512, 256, "tiny_b4");
    check_case(32, 4096, 18992, 132944, 0, 256, "shard8_b32");
    // parity cases meant for the row-streaming kernel
    check_case(33, 512, 3001, 16, 64, 256, "rows_b33");
    check_case(40, 4096, 3000, 0, 128, 256, "rows_b40");
    check_case(100, 512, 3001, 0, 64, 256, "rows_b100");
    check_case(128, 512, 70000, 32, 2048, 256, "rows_b128");
    check_case(100, 512, 102400, 0, 4096, 256, "rows_b100_tail144");
    check_case(150, 256, 2000, 0, 128, 256, "rows_b150");
    check_case(256, 256, 70000, 0, 4096, 256, "rows_b256");
    check_case(300, 256, 5000, 0, 64, 256, "rows_b300");
    check_case(200, 512, 30000, 0, 128, 256, "rows_b200_d512");

    // a grid of shapes, extremes included
    const int Bs[] = {1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257,
                      1000, 4096, 65536, kMaxB};
    const int ds[] = {8, 64, 136, 256, 512, 1024, 2048, 4096, 5120, 8192, 1 << 16, 1 << 20};
    const int Vs[] = {1, 15, 16, 17, 40, 64, 1000, 4096, 151936, 152064, 1 << 20, 1 << 26,
                      INT32_MAX - 16, INT32_MAX};
    const int tiles[] = {0, 16, 48, 128, 19008, 1 << 30};
    const int cuss[] = {1, 8, 80, 256, 304};
    for (int B : Bs)
        for (int d : ds)
            for (int V : Vs)
                for (int tv : tiles)
                    for (int cus : cuss) {
                        if ((int64_t)B * d > (int64_t)1 << 36) continue;   // H past 128 GiB
                        check_case(B, d, V, 0, tv, cus, nullptr);
                    }
    // ids offset to the end of the int32 range
    for (int V : {16, 1000, 151936})
        check_case(32, 4096, V, (INT32_MAX - V) / 16 * 16, 0, 256, nullptr);
    if (g_fail) {
        std::printf("failures %d of %ld cases\n", g_fail, g_cases);
        return 1;
    }
    std::printf("ok %ld cases, %ld reported unsupported\n", g_cases, g_unlaunchable);
    return 0;
}
