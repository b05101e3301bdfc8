// fa_bwd_kernel.hip -- attention backward pass for gfx950 (MI355X, CDNA4):
// the entry point and the D = 128 instances.  The method and its mapping
// onto CDNA4 are described in fa_bwd_kernels.h (page "TileLang 与机器学习训练：
// 反向传播算子优化案例", section "算子拆分与流水线设计").
#include "fa_bwd_kernels.h"

namespace fa {

int launch_backward(const BwdProblem &p, hipStream_t stream)
{
    // per-lane tile offsets are 32-bit: the tallest staged tile, 256 rows
    // (the dK/dV kernel's V rows), of the widest tensor must span < 2 GiB
    if ((int64_t)p.H * p.D * 2 * 256 > 0x7fffffff) return FA_ERR_SHAPE;
    bwd::BwdArgs a;
    a.q = (const _Float16 *)p.q;
    a.k = (const _Float16 *)p.k;
    a.v = (const _Float16 *)p.v;
    a.o = (const _Float16 *)p.o;
    a.dout = (const _Float16 *)p.dout;
    a.lse = p.lse;
    a.delta = p.delta;
    a.dq = (_Float16 *)p.dq;
    a.dk = (_Float16 *)p.dk;
    a.dv = (_Float16 *)p.dv;
    a.Lq = p.Lq;
    a.Lk = p.Lk;
    a.past_len = p.causal ? p.past_len : 0;
    a.H = p.H;
    a.Hkv = p.Hkv;
    a.groups = p.H / p.Hkv;
    a.n_blocks_item = 0;
    a.n_items = 0;
    a.n_rows = (int64_t)p.B * p.Lq * p.H;
    a.scale = p.scale;
    a.c = p.scale * bwd::kLog2e;
    if (p.D == 64) return bwd::launch_backward_d64(a, p.B, p.causal, stream);
    return p.causal ? bwd::launch_bwd<128, true>(a, p.B, stream) : bwd::launch_bwd<128, false>(a, p.B, stream);
}

}  // namespace fa
