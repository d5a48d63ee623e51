"""One FSDP unit with TIDE's collectives in place of FSDP2's layout copies.

FSDP2 keeps every parameter (and its gradient) as its own tensor, while its
collectives work on one flat rank-major buffer, so each step packs the
gradients into that buffer before the reduce-scatter and copies the
all-gathered buffer back out into the parameters ("FSDP通信终局：TIDE零拷贝
集合通信优化", §"FSDP2通信开销的根源").  TIDE folds both layout changes into
the collectives' addressing (§"TIDE的设计思路").  TideUnit holds one unit's
state laid out that way on one device, for N ranks:

    master   [N, S] fp32   rank r's shard of the master weights = row r
    grad     [N, S] fp32   rank r's reduced gradient shard = row r
    gathered [N*S]  bf16   the all-gather buffer (rank-major)
    params   P tensors     the unsharded parameters, each its own tensor

reduce_scatter() runs tide_rs for every rank straight from the per-parameter
gradients (fp32 reduction, the mean by default: tqpw.cn "FSDP技术演进全景图"
§3.2 reduces in fp32; apxml "Communication volume analysis" §"分片中的通信
原语" averages).  all_gather() casts the master shards into the gathered
buffer and places it with tide_ag.  The optimizer updates `master` from
`grad` in between, shard by shard.  With all N ranks in one device's memory
this is one GPU's emulation of the data-parallel group; across GPUs each
rank would hold only its rows and its peers' blocks would arrive over the
network.
"""
import contextlib

import torch

from . import Plan, ag, grad_table, pack, rs


class TideUnit:
    def __init__(self, shapes, world, device="cuda", align=1, param_dtype=torch.bfloat16):
        self.plan = Plan(shapes, world, align)
        N, S = world, self.plan.S
        self.shapes = [tuple(s) for s in shapes]
        self.world = N
        self.param_dtype = param_dtype
        self.master = torch.zeros(N, S, dtype=torch.float32, device=device)
        self.grad = torch.zeros(N, S, dtype=torch.float32, device=device)
        self.gathered = torch.zeros(N * S, dtype=param_dtype, device=device)
        self.params = [torch.empty(s, dtype=param_dtype, device=device) for s in self.shapes]

    def load(self, full):
        """Shard full fp32 tensors into the master rows (tide_pack of 4-byte
        elements; padding stays 0) and place them into `params`."""
        tensors = [t.detach().to(device=self.master.device, dtype=torch.float32).contiguous()
                   for t in full]
        pack(self.plan, tensors, self.master.view(-1))
        self.all_gather()

    def reduce_scatter(self, grads, avg=True, small=False, stream=None):
        """grads[r][i] = rank r's gradient of parameter i (bf16, fp16 or fp32,
        one dtype): row r of `grad` becomes rank r's reduced shard."""
        table = grad_table(self.plan, grads)
        for R in range(self.world):
            rs(self.plan, R, table, self.grad[R], small=small, avg=avg, stream=stream)

    def all_gather(self, small=False, copy_engine=False, stream=None):
        """Master shards -> param dtype into the gathered buffer -> params."""
        with torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext():
            self.gathered.view(self.world, self.plan.S).copy_(self.master)
        ag(self.plan, self.gathered, self.params, small=small, copy_engine=copy_engine,
           stream=stream)

