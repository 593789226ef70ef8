"""TEST INFRASTRUCTURE: execute a whole-node relay schedule on the host, every
hop a numpy copy and every local step the CPU oracle's function for it."""
import numpy as np

import oracle as orc
from pack_rr_helper_amd.schedule import NODE


def run_on_cpu(s, inputs):
    npdt = inputs[0].dtype
    buf = {key: np.zeros(n, npdt) for key, n in s.buffers.items()}
    for r in range(NODE):
        buf[(r, "in")][:] = inputs[r]

    def view(ref):
        return buf[(ref.rank, ref.buf)][ref.off:ref.off + ref.n]

    dt = s.dtype
    es = 4 if dt == orc.F32 else 2
    for grp in s.groups:
        for h in grp.hops:
            if not h.via:
                view(h.dst)[:] = view(h.src)
        for st in grp.after:
            r = st.relay
            if st.kind == "copy":
                view(st.outs[0])[:] = view(st.ins[0])
            elif st.kind == "helper_reduce":
                ins = [view(x).copy() for x in st.ins]
                res = orc.ar2_helper(dt, s.op, *ins) if r.A == 2 else orc.ar4_helper(dt, s.op, ins)
                view(st.outs[0])[:] = res
            elif st.kind == "active" and st.coll == orc.ALLREDUCE:
                ins = [view(x).copy() for x in st.ins]
                out = view(st.outs[0])
                tmp = out.copy()
                orc.ar_active(dt, s.op, r.A, r.H, r.numChunks, r.permille, r.count, st.idx, ins, tmp)
                out[:] = tmp
            elif st.kind == "active":
                view(st.outs[0])[:] = orc.rs2_active(dt, s.op, view(st.ins[0]).copy(), view(st.ins[1]).copy())
            elif st.kind == "rs_pass1":
                c = st.outs[0].n // r.A
                view(st.outs[0])[:] = orc.rs4_pass1(dt, r.A, c, view(st.ins[0]).copy())
            elif st.kind == "rs_pass2":
                blocks = [view(x).copy() for x in st.ins[:r.A]]
                reds = [view(x).copy() for x in st.ins[r.A:]]
                view(st.outs[0])[:] = orc.rs4_pass2(dt, s.op, r.A, r.H, r.permille, r.count, st.idx, blocks, reds)
            elif st.kind == "a2a_pack":
                c = st.outs[0].n // (r.A - 1)
                dst = orc.a2a_pack(es, r.A, r.count, c, st.idx, [view(x).copy() for x in st.ins])
                for o, d in zip(st.outs, dst):
                    view(o)[:] = d.view(npdt)
            elif st.kind == "a2a_unpack":
                c = st.ins[0].n // (r.A - 1)
                outs = [view(o) for o in st.outs]
                tmp = [o.copy() for o in outs]
                orc.a2a_unpack(es, r.A, r.count, c, st.idx, [view(x).copy() for x in st.ins], tmp)
                for o, t in zip(outs, tmp):
                    o[:] = t
            else:
                raise ValueError(st.kind)
    return [buf[(r, "out")] for r in range(NODE)]
