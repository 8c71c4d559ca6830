// Host program for the GEMM schedule rules (blockwise_scaled_fp8_act_amd/csrc/schedule.hpp, the
// header the library calls before each GEMM launch). Reads one query per line from stdin and
// prints one answer per line:
//   plan M N K fnuz cus max_bytes            -> S bm bn bytes
//   forced M N K cus S bm bn max_bytes       -> S bm bn bytes
//   stages bn per_col wgs cus                -> stages
//   lhs M Kb cus                             -> pieces per thread of quantize_lhs's row strips
//   maxstages bn per_col                     -> the thin kernel's deepest pipeline that fits the LDS
//   waves bn wgs cus                         -> the thin kernel's waves per workgroup
//   colsplit M N K cus max_bytes             -> n1 S bytes of the column split (n1 0: none)
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <iostream>
#include <sstream>
#include <string>

#include "schedule.hpp"

int main() {
    std::string line;
    while (std::getline(std::cin, line)) {
        std::istringstream in(line);
        std::string kind;
        in >> kind;
        if (kind == "plan") {
            int64_t M, N, K, maxb;
            int fnuz, cus;
            in >> M >> N >> K >> fnuz >> cus >> maxb;
            const bsfp8::SplitPlan p = bsfp8::gemm_split_plan(M, N, K, fnuz != 0, cus, maxb);
            std::printf("%d %d %d %lld\n", p.S, p.bm, p.bn, (long long)p.bytes);
        } else if (kind == "forced") {
            int64_t M, N, K, maxb;
            int cus, S, bm, bn;
            in >> M >> N >> K >> cus >> S >> bm >> bn >> maxb;
            const bsfp8::SplitPlan p = bsfp8::gemm_split_plan_forced(M, N, K, false, cus, S, bm, bn, maxb);
            std::printf("%d %d %d %lld\n", p.S, p.bm, p.bn, (long long)p.bytes);
        } else if (kind == "stages") {
            int bn, per_col, cus;
            int64_t wgs;
            in >> bn >> per_col >> wgs >> cus;
            std::printf("%d\n", bsfp8::sched::thin_stages(bn, per_col != 0, wgs, cus));
        } else if (kind == "colsplit") {
            int64_t M, N, K, maxb;
            int cus;
            in >> M >> N >> K >> cus >> maxb;
            const bsfp8::ColumnSplit c = bsfp8::gemm_column_split(M, N, K, cus, maxb);
            std::printf("%lld %d %lld\n", (long long)c.n1, c.tail.S, (long long)c.tail.bytes);
        } else if (kind == "waves") {
            int bn, cus;
            int64_t wgs;
            in >> bn >> wgs >> cus;
            std::printf("%d\n", bsfp8::sched::thin_waves(bn, wgs, cus));
        } else if (kind == "maxstages") {
            int bn, per_col;
            in >> bn >> per_col;
            std::printf("%d\n", bsfp8::sched::thin_max_stages(bn, per_col != 0));
        } else if (kind == "lhs") {
            int64_t M, Kb;
            int cus;
            in >> M >> Kb >> cus;
            std::printf("%d\n", bsfp8::sched::lhs_strip_loads(M, Kb, cus));
        } else {
            std::printf("?\n");
        }
        std::fflush(stdout);
    }
    return 0;
}
