// plan_fuzz.cpp -- randomized checks of the host planner, built with
// AddressSanitizer and UndefinedBehaviorSanitizer by test_plan_sanitizers.py
// (host code only; no HIP call is made). Every plan that validates must tile
// its work exactly: tile counts follow the part/segment sizes, tile ranges
// are monotone, and launch shapes are within the kernels' limits.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>

#include "../reduce_atom_03_amd/csrc/plan.hpp"

using namespace atom;

namespace {

int fails = 0;

void check(bool ok, const char* what, int iter)
{
    if (!ok) {
        std::fprintf(stderr, "iteration %d: %s\n", iter, what);
        ++fails;
    }
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

void check_reduce(const Plan& p, int iter)
{
    const ReduceArgs& a = p.ra;
    const int64_t ve = kVecBytes / p.esize;
    const int64_t ts = static_cast<int64_t>(p.wg) * p.U;
    check(a.nparts >= 1 && a.nparts <= kMaxRanks, "reduce nparts", iter);
    check(p.wg == 64 || p.wg == 128 || p.wg == 256, "reduce wg", iter);
    check(p.vec ? (p.U == 1 || p.U == 2 || p.U == 4) : p.U == 1, "reduce U", iter);
    check(p.U * a.nsrc <= 32 || p.U == 1, "reduce registers", iter);
    int64_t t = 0;
    for (int k = 0; k < a.nparts; ++k) {
        check(a.tile_begin[k] == t, "reduce tile_begin", iter);
        const int64_t len = a.part_off[k + 1] - a.part_off[k];
        check(len >= 0, "reduce part length", iter);
        const int64_t shift = p.vec ? a.shift[k] : 0;
        check(shift >= 0 && shift < ts, "reduce shift", iter);
        const int64_t h = a.head[k];
        check(h >= 0 && h < ve && h <= len && (p.vec || h == 0), "reduce head", iter);
        int64_t tiles = cdiv(cdiv(len - h, ve) + shift, ts);
        if (h > 0 && tiles == 0)
            tiles = 1;
        if (a.shifted && len > 0) {
            // shifted path: the part's aligned source vectors plus one
            check(p.vec && h == 0 && shift == 0, "reduce shifted shape", iter);
            const uint64_t a0 = reinterpret_cast<uintptr_t>(a.src[0]) + static_cast<uint64_t>(a.part_off[k] * p.esize);
            const int64_t vlo = static_cast<int64_t>(a0 / kVecBytes);
            const int64_t nv = static_cast<int64_t>((a0 + len * p.esize - 1) / kVecBytes) + 2 - (vlo & ~(ts - 1));
            tiles = cdiv(nv, ts);
        }
        t += tiles;
    }
    check(a.tile_begin[a.nparts] == t && a.ntiles == t, "reduce ntiles", iter);
    check(p.grid >= 1 && p.grid <= std::max<int64_t>(1, t), "reduce grid", iter);
}

void check_copy(const Plan& p, int iter)
{
    const CopyArgs& a = p.ca;
    check(a.tile_bytes == static_cast<int64_t>(p.wg) * p.U * kVecBytes, "copy tile bytes", iter);
    check(a.nseg >= 1 && a.nseg <= kMaxSegs, "copy nseg", iter);
    int64_t t = 0;
    for (int s = 0; s < a.nseg; ++s) {
        check(a.seg_tile_begin[s] == t, "copy seg_tile_begin", iter);
        check(a.cnt[s] >= 0, "copy count", iter);
        const int64_t h = a.head[s];
        const int64_t bytes = static_cast<int64_t>(a.cnt[s]) * a.row_bytes - h;
        check(h >= 0 && h < kVecBytes && bytes >= 0 && (p.vec || h == 0), "copy head", iter);
        // an aligned segment may need one extra (short) tile at its start; a
        // segment that is all head has one tile
        const int64_t lo = std::max<int64_t>(cdiv(bytes, a.tile_bytes), h > 0 ? 1 : 0);
        // (a shifted segment also covers one vector past its end and may
        // start up to a tile before its first)
        const int64_t hi = bytes ? cdiv(bytes, a.tile_bytes) + (a.shifted ? 2 : 1) : lo;
        const int64_t n = (s + 1 <= a.nseg ? a.seg_tile_begin[s + 1] : 0) - a.seg_tile_begin[s];
        check(n >= lo && n <= hi, "copy tiles per segment", iter);
        t = a.seg_tile_begin[s + 1];
    }
    check(a.ntiles == t, "copy ntiles", iter);
    if (a.block_shift >= 0) {
        // blocked fan-out: (block, output, tile) workgroup tasks, a grid
        // stride that keeps every workgroup on one XCD
        check(a.kind == CK_FANOUT && a.ndst > 1 && a.grid_segs == 0 && a.nseg <= kMaxRanks,
              "copy blocked kind", iter);
        check(a.block_shift >= 3 && a.block_shift <= 30, "copy block shift", iter);
        const int64_t bt = int64_t(1) << a.block_shift;
        check(a.nwork == cdiv(t, bt) * bt * a.ndst && (a.nwork >> a.block_shift) <= 0xFFFFFFFFll,
              "copy blocked tasks", iter);
        check(p.grid >= 1 && p.grid <= std::min<int64_t>(a.nwork, kMaxGridBlocked), "copy blocked grid", iter);
        int64_t off = 0;
        for (int s = 0; s < a.nseg; ++s) {
            check(a.seg_off[s] == off, "copy blocked offsets", iter);
            off += static_cast<int64_t>(a.cnt[s]) * a.row_bytes;
        }
        check(a.seg_off[a.nseg] == off, "copy blocked size", iter);
    } else {
        check(p.grid >= 1 && p.grid <= std::max<int64_t>(1, t), "copy grid", iter);
    }
}

}  // namespace

int main(int argc, char** argv)
{
    const int iters = argc > 1 ? std::atoi(argv[1]) : 20000;
    std::mt19937_64 rng(12345);
    auto pick = [&](int64_t lo, int64_t hi) {
        return std::uniform_int_distribution<int64_t>(lo, hi)(rng);
    };
    int ok_plans = 0;
    for (int iter = 0; iter < iters; ++iter) {
        const bool valid_pair = pick(0, 9) < 7;             // mostly collectives that exist
        const int P = static_cast<int>(valid_pair ? pick(1, 16) : pick(0, 18));
        static const int pairs[4][3] = {{0, 1, 1}, {1, 2, 0}, {0, 3, 0}, {0, 2, 1}};
        const int* pr = pairs[pick(0, 3)];
        const atom_layout_kind kin = static_cast<atom_layout_kind>(valid_pair ? pr[0] : pick(-1, 4));
        const atom_layout_kind kout = static_cast<atom_layout_kind>(valid_pair ? pr[1] : pick(0, 4));
        const atom_op op = static_cast<atom_op>(valid_pair ? pr[2] : pick(-1, 2));
        const atom_dtype dt = static_cast<atom_dtype>(valid_pair ? pick(0, 1) : pick(-1, 2));
        void* ins[32];
        void* outs[32];
        const uint64_t base_in = 0x100000000000ull, base_out = 0x200000000000ull;
        const uint64_t stride = 1ull << 36;                 // buffers never overlap
        const int misalign = pick(0, 7) == 0 ? static_cast<int>(pick(1, 15)) : 0;
        for (int r = 0; r < 32; ++r) {
            ins[r] = reinterpret_cast<void*>(base_in + r * stride + (r == 1 ? misalign : 0));
            outs[r] = reinterpret_cast<void*>(base_out + r * stride);
        }
        int64_t counts[kMaxSegs + 8];
        const bool v = pick(0, 2) == 0;
        for (auto& c : counts)
            c = pick(0, 49) == 0 ? pick(-3, 0) : pick(0, 5000);
        const int64_t n = pick(0, 4) == 0 ? pick(-2, 40) : pick(0, 1 << 22);
        atom_layout li{kin, P, ins, n, v ? counts : nullptr, pick(0, 9) == 0 ? 0 : pick(1, 7168), dt};
        atom_layout lo{kout, P, outs, n, nullptr, li.row_elems, dt};
        atom_config cfg{};
        const bool use_cfg = pick(0, 1) == 1;
        if (use_cfg) {
            cfg.chunk_bytes = pick(0, 3) == 0 ? pick(-1, 1 << 25) : (int64_t(1) << pick(16, 24));
            cfg.stages = static_cast<int32_t>(pick(0, 4) == 0 ? pick(-1, 9) : (1 << pick(0, 3)));
            cfg.num_wgs = static_cast<int32_t>(pick(0, 2) == 0 ? pick(-2, 3000) : 0);
            cfg.flags = static_cast<uint32_t>(pick(0, 8));
            cfg.ring_slots = static_cast<int32_t>(pick(0, 3) == 0 ? pick(-1, 70) : 0);
            cfg.piece_bytes = static_cast<int32_t>(pick(0, 3) == 0 ? (1 << pick(13, 22)) : 0);
            cfg.wait_us = static_cast<int32_t>(pick(0, 5) == 0 ? pick(-1, 10) : 0);
            static const int32_t lanes[] = {0, 64, 128, 256, 0, 32, 100, 512, 1024, 2048};
            cfg.lanes = lanes[pick(0, 9)];
        }
        Plan p;
        const atom_status st = plan_collective(&li, &lo, op, use_cfg ? &cfg : nullptr, &p);
        check(st == ATOM_OK || st == ATOM_ERR_INVALID_ARG || st == ATOM_ERR_UNSUPPORTED,
              "status", iter);
        if (st != ATOM_OK)
            continue;
        ++ok_plans;
        check(p.P == P && P >= 1 && P <= kMaxRanks, "ranks", iter);
        check(p.credited_bytes >= 0, "credited bytes", iter);
        if (p.exec == EX_REDUCE)
            check_reduce(p, iter);
        else if (p.exec == EX_COPY)
            check_copy(p, iter);
        else if (p.exec == EX_SNAC_COPY || p.exec == EX_SNAC_REDUCE) {
            check(p.sa.slots >= 1 && p.sa.slots <= kMaxSlots, "snac slots", iter);
            check(p.sa.pieces >= 1 && p.sa.piece_bytes * p.sa.pieces == p.sa.chunk_bytes,
                  "snac pieces", iter);
            check(p.sa.ntasks == 2 * p.sa.nchunks * p.sa.pieces, "snac tasks", iter);
            check(p.sa.slot_bytes == p.sa.chunk_bytes + kSlotPad &&
                      p.ring_bytes == p.sa.slot_bytes * p.sa.slots, "snac ring", iter);
            for (int s = 0; s < p.sa.nseg; ++s)
                check(p.sa.head[s] < kVecBytes && p.sa.elem[s] <= SE_SHIFT &&
                          (p.sa.elem[s] != SE_ELEM || p.sa.head[s] == 0) &&
                          p.sa.head[s] % p.esize == 0,
                      "snac segment offset", iter);
            check(p.wg >= 64 && p.wg <= 512 && p.wg % 64 == 0, "snac wg", iter);
            check(!use_cfg || cfg.lanes == 0 || p.wg == cfg.lanes, "snac lanes", iter);
        }
    }
    // a few copies and flat reduces
    for (int iter = 0; iter < iters / 10; ++iter) {
        Plan p;
        const size_t bytes = static_cast<size_t>(pick(0, 1 << 26));
        void* d = reinterpret_cast<void*>(0x300000000000ull + pick(0, 15));
        const void* s = reinterpret_cast<const void*>(0x400000000000ull + pick(0, 15));
        if (plan_copy(d, s, bytes, nullptr, &p) == ATOM_OK && p.exec == EX_COPY)
            check_copy(p, iter);
        const void* srcs[kMaxRanks];
        for (int r = 0; r < kMaxRanks; ++r)
            srcs[r] = reinterpret_cast<const void*>(0x500000000000ull + r * (1ull << 34));
        const int nsrc = static_cast<int>(pick(1, 16));
        if (plan_reduce(d, srcs, nsrc, pick(0, 1 << 22), ATOM_DT_F32, ATOM_OP_SUM, nullptr, &p) ==
                ATOM_OK && p.exec == EX_REDUCE)
            check_reduce(p, iter);
    }
    // MoE routing and movement plans
    int ok_moe = 0;
    for (int iter = 0; iter < iters / 4; ++iter) {
        const bool sane = pick(0, 9) < 7;
        const int P = static_cast<int>(sane ? pick(1, 16) : pick(-1, 18));
        const int per = static_cast<int>(pick(1, 64));
        const int E = sane ? P * per : static_cast<int>(pick(-1, 1100));
        const int k = static_cast<int>(sane ? pick(1, 16) : pick(-1, 18));
        const int64_t T = sane ? pick(0, 3000) : pick(-2, (1 << 21));
        void* ids[kMaxRanks + 2];
        void* pos[kMaxRanks + 2];
        void* xs[kMaxRanks + 2];
        void* outs[kMaxRanks + 2];
        void* ws[kMaxRanks + 2];
        const uint64_t stride = 1ull << 36;
        const int mis = pick(0, 9) == 0 ? static_cast<int>(pick(1, 15)) : 0;
        for (int r = 0; r < kMaxRanks + 2; ++r) {
            ids[r] = reinterpret_cast<void*>(0x600000000000ull + r * stride);
            pos[r] = reinterpret_cast<void*>(0x610000000000ull + r * stride);
            xs[r] = reinterpret_cast<void*>(0x620000000000ull + r * stride + (r == 0 ? mis : 0));
            outs[r] = reinterpret_cast<void*>(0x630000000000ull + r * stride);
            ws[r] = reinterpret_cast<void*>(0x640000000000ull + r * stride);
        }
        atom_moe_routing rt{};
        rt.nranks = P;
        rt.num_experts = E;
        rt.topk = k;
        rt.reserved = pick(0, 19) == 0 ? 1 : 0;
        rt.tokens = T;
        rt.expert_ids = reinterpret_cast<const int32_t* const*>(ids);
        rt.positions = reinterpret_cast<int32_t* const*>(pos);
        rt.counts = reinterpret_cast<int32_t*>(0x650000000000ull);
        rt.recv_rows = reinterpret_cast<int64_t*>(0x660000000000ull);
        rt.scratch = reinterpret_cast<void*>(0x670000000000ull + (pick(0, 19) == 0 ? 4 : 0));
        MoeRoutePlan rp;
        if (plan_moe_route(&rt, &rp) == ATOM_OK) {
            ++ok_moe;
            const int64_t n = T * k;
            check(rp.a.nch >= 1 && static_cast<int64_t>(rp.a.nch) * kMoeChunk >= n &&
                      (n == 0 || static_cast<int64_t>(rp.a.nch - 1) * kMoeChunk < n),
                  "moe chunks", iter);
            check(rp.scan_threads >= E && rp.scan_threads <= 1024 && rp.scan_threads % 64 == 0,
                  "moe scan threads", iter);
            check(moe_scratch_bytes(P, E, k, T) >= static_cast<int64_t>(P) * rp.a.nch * E * 4,
                  "moe scratch", iter);
            check(rp.a.per * P == E, "moe experts per rank", iter);
            check(rp.a.groups >= 1 && rp.a.groups <= rp.a.nch && rp.a.groups * P <= 1024,
                  "moe placing groups", iter);
            check(rp.small == (n <= kMoeSmallEntries &&
                               (int64_t(P) * E + E + 64 * P) * 4 <= kMoeSmallLds),
                  "moe small routing", iter);
        }
        const int64_t cap = pick(0, 9) == 0 ? pick(-1, 3) : pick(0, 40000);
        const int64_t row = pick(0, 9) == 0 ? pick(-1, 9) : (pick(0, 3) == 0 ? pick(1, 8191) : 8 * pick(1, 1024));
        const atom_dtype dt = static_cast<atom_dtype>(pick(0, 9) == 0 ? pick(-1, 2) : pick(0, 1));
        for (int combine = 0; combine < 2; ++combine) {
            MoeMovePlan mp;
            atom_config mc{};
            const bool mcfg = pick(0, 2) == 0;
            if (mcfg) {
                static const int32_t mlanes[] = {0, 64, 128, 256, 512, 100};
                mc.lanes = mlanes[pick(0, 5)];
                mc.stages = static_cast<int32_t>(pick(0, 4) == 0 ? pick(-1, 9) : (1 << pick(0, 3)));
                mc.num_wgs = static_cast<int32_t>(pick(0, 2) == 0 ? pick(-2, 3000) : 0);
                mc.flags = static_cast<uint32_t>(pick(0, 8));
            }
            const atom_status ms = plan_moe_move(&rt, combine != 0, xs,
                                                 reinterpret_cast<const float* const*>(ws), outs, cap,
                                                 row, dt, mcfg ? &mc : nullptr, &mp);
            check(ms == ATOM_OK || ms == ATOM_ERR_INVALID_ARG || ms == ATOM_ERR_UNSUPPORTED,
                  "moe status", iter);
            if (ms != ATOM_OK)
                continue;
            ++ok_moe;
            const int64_t ntok = static_cast<int64_t>(P) * T;
            check(mp.wg >= 64 && mp.wg <= 256 && mp.wg % 64 == 0, "moe lanes", iter);
            check(mp.U == 1 || mp.U == 2 || mp.U == 4 || mp.U == 8, "moe U", iter);
            if (mp.a.elem) {
                // element-wise: one tile per token row
                check(mp.U == 1 && mp.a.piece_bytes == mp.a.row_bytes && mp.a.pieces == (mp.a.row_bytes > 0),
                      "moe elem piece", iter);
                check(mp.a.row_bytes % (dt == ATOM_DT_BF16 ? 2 : 4) == 0, "moe elem rows", iter);
            } else {
                check(mp.a.piece_bytes == static_cast<int64_t>(mp.wg) * mp.U * kVecBytes, "moe piece", iter);
            }
            check(ntok == 0 || mp.a.row_bytes == 0 ||
                      (mp.a.pieces * mp.a.piece_bytes >= mp.a.row_bytes &&
                       (mp.a.pieces - 1) * mp.a.piece_bytes < mp.a.row_bytes),
                  "moe pieces cover the row", iter);
            check(mp.a.ntiles == ntok * mp.a.pieces, "moe tiles", iter);
            check(mp.a.ntiles == 0 || (mp.grid >= 1 && mp.grid <= mp.a.ntiles), "moe grid", iter);
            check(mp.a.ntiles == 0 || mp.a.elem || mp.a.row_bytes % kVecBytes == 0, "moe row alignment", iter);
            check(mp.a.k == k && mp.a.per * P == E, "moe shape", iter);
            check(mp.credited_bytes == ntok * ((k + 1) * mp.a.row_bytes + k * (combine ? 12 : 8)),
                  "moe credited bytes", iter);
        }
    }
    std::printf("%d MoE plans validated\n", ok_moe);
    std::printf("%d plans validated, %d failures\n", ok_plans, fails);
    return fails ? 1 : 0;
}
