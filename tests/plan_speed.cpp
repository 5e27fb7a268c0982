// plan_speed.cpp -- host cost of planning a call (validation, collective
// derivation, tiles), built with g++ -O2 by test_plan_speed.py: the decode
// AllReduce of 8 x b x 7168 bf16 (b = 1 and 16) and the AllToAllV of
// 8 x 4096 rows, each planned many times; prints ns per plan.
#include <chrono>
#include <cstdint>
#include <cstdio>
#include <initializer_list>

#include "../reduce_atom_03_amd/csrc/plan.hpp"

using namespace atom;

// The best of 7 repeats of `iters` plans: planning is deterministic, so the
// fastest repeat is its cost and slower ones measure interference from other
// processes on the host.
static double time_plan(const atom_layout& in, const atom_layout& out, atom_op op, int iters)
{
    Plan p;
    int64_t sink = 0;
    double best = 1e30;
    for (int rep = 0; rep < 7; ++rep) {
        const auto t0 = std::chrono::steady_clock::now();
        for (int i = 0; i < iters; ++i) {
            if (plan_collective(&in, &out, op, nullptr, &p) != ATOM_OK)
                return -1.0;
            sink += p.grid;
        }
        const auto t1 = std::chrono::steady_clock::now();
        const double ns = std::chrono::duration<double, std::nano>(t1 - t0).count() / iters;
        best = ns < best ? ns : best;
    }
    if (sink == 42)
        std::printf("#");
    return best;
}

int main()
{
    void* ins[8];
    void* outs[8];
    for (int r = 0; r < 8; ++r) {
        ins[r] = reinterpret_cast<void*>(0x100000000000ull + (uint64_t(r) << 36));
        outs[r] = reinterpret_cast<void*>(0x200000000000ull + (uint64_t(r) << 36));
    }
    const int iters = 40000;
    for (int b : {1, 16}) {
        const int64_t n = int64_t(b) * 896;     // b x 7168 elements in 8 partitions
        atom_layout li{ATOM_LAYOUT_PARTITIONED, 8, ins, n, nullptr, 1, ATOM_DT_BF16};
        atom_layout lo{ATOM_LAYOUT_GATHERED, 8, outs, n, nullptr, 1, ATOM_DT_BF16};
        std::printf("allreduce_b%d %.1f\n", b, time_plan(li, lo, ATOM_OP_SUM, iters));
    }
    int64_t C[64];
    for (int i = 0; i < 64; ++i)
        C[i] = 64 + (i * 37) % 900;
    atom_layout li{ATOM_LAYOUT_PARTITIONED, 8, ins, 0, C, 7168, ATOM_DT_BF16};
    atom_layout lo{ATOM_LAYOUT_TRANSPOSED, 8, outs, 0, nullptr, 7168, ATOM_DT_BF16};
    std::printf("alltoallv %.1f\n", time_plan(li, lo, ATOM_OP_COPY, iters));
    return 0;
}
