"""A small CPU interpreter for the gfx950 instructions the weights-in-code generator emits.

Test infrastructure: it runs the generated kernel of a packed layer on the host, wavefront
by wavefront, so that the CPU suite can compare the generated code with the oracle without
a GPU.  It executes exactly the instruction forms the generator writes and rejects anything
else, and it checks the rules the hardware does not check for the code:

  * the wait states gfx950 needs and does not enforce itself (as its compiler's hazard
    recognizer inserts them): a DPP read of a VGPR two after a VALU write of it or the issue
    of a load into it, v_readfirstlane of a VGPR one after a VALU write of it, and a VALU
    read of VCC two after a VALU write of VCC;
  * a VGPR that an outstanding buffer load will write may not be read or written before an
    s_waitcnt vmcnt has retired that load (buffer loads and stores, LDS DMA included, report
    completion in the order they were issued, so vmcnt(n) retires the oldest until n remain;
    issuing a 64th outstanding operation waits for the oldest, as the hardware stalls the
    issue at the counter's limit), and likewise a VGPR an outstanding LDS instruction
    (ds_read, ds_bpermute) will write before s_waitcnt lgkmcnt;
  * only VGPRs below the kernel's declared count are used;
  * every output element is stored at most once per launch.

Buffer loads and stores follow the raw-buffer rules the kernel relies on: an access whose
offset (vector offset plus scalar offset) is at or past the descriptor's byte range loads
zero or is dropped.  Floating-point FMAs are evaluated in double precision and rounded once
to fp32 (a fused fp32 FMA rounds the exact a*b + c once; the double sum can differ from it
only by a double rounding, far inside the comparison tolerance).
"""
from __future__ import annotations

import re
import struct

import numpy as np

_REG = re.compile(r"^([sv])(\d+)$")
_RANGE = re.compile(r"^([sv])\[(\d+):(\d+)\]$")


class EmuError(AssertionError):
    pass


def _u32(x):
    return np.uint32(x & 0xFFFFFFFF)


class Kernel:
    """Parsed code of one generated kernel (the text before its descriptor)."""

    def __init__(self, src: str):
        code = src.split("\t.section .rodata")[0]
        self.instrs = []
        self.labels = {}
        for raw in code.splitlines():
            line = raw.strip()
            if not line or line.startswith("."):
                if line.endswith(":"):
                    self.labels[line[:-1]] = len(self.instrs)
                continue
            if line.endswith(":"):
                self.labels[line[:-1]] = len(self.instrs)
                continue
            op, _, rest = line.partition(" ")
            args = [a.strip() for a in re.split(r",(?![^\[]*\])", rest)] if rest else []
            self.instrs.append((op, args))
        m = re.search(r"\.amdhsa_next_free_vgpr (\d+)", src)
        self.nvgpr = int(m.group(1))
        m = re.search(r"\.amdhsa_next_free_sgpr (\d+)", src)
        self.nsgpr = int(m.group(1))
        m = re.search(r"\.amdhsa_group_segment_fixed_size (\d+)", src)
        self.lds_bytes = int(m.group(1))


class Wave:
    def __init__(self, kern: Kernel, kernarg: bytes, wg_id: int, wave_in_wg: int, bufs, lds=None, lds_pend=None):
        self.k = kern
        self.lds = lds  # the workgroup's LDS (uint32 words), shared by its waves
        self.lds_pend = lds_pend  # per LDS word: an LDS DMA into it is not yet retired (vmcnt)
        self.m0 = None
        self.m0_wr = -100  # instruction count at the last write of m0
        self.barriers = 0  # s_barrier instructions executed
        self.lgkm = []  # per outstanding LDS instruction (oldest first): the VGPRs it writes
        self.s = np.zeros(110, np.uint64)  # scalar registers (kept as u32 values)
        self.v = np.zeros((256, 64), np.uint32)
        self.vcc = np.zeros(64, bool)
        self.scc = False
        self.kernarg = kernarg
        self.bufs = bufs  # list of (base address, numpy uint32 view) for x and y
        self.s[2] = wg_id
        self.v[0] = np.arange(64, dtype=np.uint32) + 64 * wave_in_wg
        self.valu = 0
        self.wr = np.full(256, -100, np.int64)
        self.vcc_wr = -100
        self.pending = []  # outstanding vector memory operations, oldest first: a load's VGPR,
                           # ("lds", words) for an LDS DMA, ("store", None) for a store
        self.stores = []   # (buffer index, element indices, values)

    # ---- operands ----
    def sreg(self, a):
        m = _REG.match(a)
        if not m or m.group(1) != "s":
            raise EmuError(f"expected an SGPR, got {a}")
        i = int(m.group(2))
        if i >= self.k.nsgpr:
            raise EmuError(f"s{i} beyond the declared {self.k.nsgpr} SGPRs")
        return i

    def vreg(self, a, write=False):
        m = _REG.match(a)
        if not m or m.group(1) != "v":
            raise EmuError(f"expected a VGPR, got {a}")
        i = int(m.group(2))
        if i >= self.k.nvgpr:
            raise EmuError(f"v{i} beyond the declared {self.k.nvgpr} VGPRs")
        if any(e == i for e in self.pending if not isinstance(e, tuple)) or any(i in regs for regs in self.lgkm):
            raise EmuError(f"v{i} {'written' if write else 'read'} while a load into it is outstanding")
        return i

    def vtuple(self, a, n):
        m = _RANGE.match(a)
        if not m or m.group(1) != "v" or int(m.group(3)) - int(m.group(2)) + 1 != n:
            raise EmuError(f"expected a {n}-register VGPR tuple, got {a}")
        lo = int(m.group(2))
        if lo % 2:
            raise EmuError(f"VGPR tuple {a} not even-aligned")
        return [self.vreg(f"v{lo + j}") for j in range(n)]

    def sval(self, a):
        """A scalar operand value (SGPR, integer constant, or a difference of two labels,
        taken in instruction slots as the emulated program counter counts them)."""
        if a.startswith("s"):
            return int(self.s[self.sreg(a)]) & 0xFFFFFFFF
        if a.startswith(".L"):
            x, y = a.split("-")
            return (self.k.labels[x] - self.k.labels[y]) & 0xFFFFFFFF
        return int(a, 0) & 0xFFFFFFFF

    def need(self, since, n, what):
        if self.valu - since - 1 < n:
            raise EmuError(f"{what}: {self.valu - since - 1} wait states, {n} needed")

    def src_vec(self, a):
        """A vector-instruction source: VGPR (per lane), SGPR or constant (broadcast)."""
        if a.startswith("v"):
            return self.v[self.vreg(a)].copy()
        return np.full(64, self.sval(a), np.uint32)

    def wv(self, a, vals):
        i = self.vreg(a, write=True)
        self.v[i] = vals.astype(np.uint32)
        self.wr[i] = self.valu
        self.valu += 1

    def rsrc(self, a):
        m = _RANGE.match(a)
        base = int(m.group(2))
        w = [int(self.s[base + j]) & 0xFFFFFFFF for j in range(4)]
        addr = w[0] | ((w[1] & 0xFFFF) << 32)
        if (w[1] >> 16) != 0 or w[3] != 0x20000:
            raise EmuError(f"unexpected descriptor {w}")
        return addr, w[2]

    def buffer(self, addr):
        for i, (base, arr) in enumerate(self.bufs):
            if base == addr:
                return i, arr
        raise EmuError(f"descriptor base {addr:#x} is no known buffer")

    def _retire(self, q):
        e = q.pop(0)
        if isinstance(e, tuple) and e[0] == "lds":  # an LDS DMA: its words are now written
            self.lds_pend[e[1]] = False

    def _issue_vmem(self, e):
        if len(self.pending) >= 63:  # the counter is full: the issue waits for the oldest
            self._retire(self.pending)
        self.pending.append(e)

    # ---- execution (a generator: yields at s_barrier) ----
    def run(self, max_steps=10_000_000):
        pc = 0
        steps = 0
        ins = self.k.instrs
        while True:
            steps += 1
            self.steps = steps
            if steps > max_steps:
                raise EmuError("too many steps")
            op, a = ins[pc]
            pc += 1
            if op == "s_endpgm":
                if self.lgkm:
                    raise EmuError("program ends with LDS reads outstanding")
                return
            if op == "s_load_dwordx8" or op == "s_load_dwordx2":
                m = _RANGE.match(a[0])
                lo, hi = int(m.group(2)), int(m.group(3))
                off = int(a[2], 0)
                n = hi - lo + 1
                vals = struct.unpack_from(f"<{n}I", self.kernarg, off)
                for j in range(n):
                    self.s[lo + j] = vals[j]
            elif op == "s_waitcnt":
                m = re.match(r"(vmcnt|lgkmcnt)\((\d+)\)", a[0])
                keep = int(m.group(2))
                q = self.pending if m.group(1) == "vmcnt" else self.lgkm
                while len(q) > keep:
                    self._retire(q)
            elif op == "s_barrier":
                if self.lgkm:
                    raise EmuError("s_barrier with LDS reads outstanding")
                self.barriers += 1
                yield "barrier"
            elif op in ("ds_write_b128", "ds_read_b128"):
                if self.lds is None:
                    raise EmuError("LDS access in a kernel without LDS")
                last, _, mods = a[1].partition(" ")
                off = 0
                if mods:
                    key, _, num = mods.partition(":")
                    if key != "offset":
                        raise EmuError(f"LDS modifier not emulated: {mods}")
                    off = int(num)
                if op == "ds_write_b128":
                    addr = self.src_vec(a[0]).astype(np.int64) + off
                    regs = self.vtuple(last, 4)
                else:
                    addr = self.src_vec(last).astype(np.int64) + off
                    regs = self.vtuple(a[0], 4)
                if (addr % 16).any() or (addr < 0).any() or (addr + 16 > self.lds.size * 4).any():
                    raise EmuError(f"{op} outside the LDS or misaligned")
                w = addr // 4
                for j in range(4):
                    if op == "ds_write_b128":
                        self.lds[w + j] = self.v[regs[j]]
                    else:
                        self.v[regs[j]] = self.lds[w + j]
                if op == "ds_read_b128":
                    self.lgkm.append(regs)
                    if len(self.lgkm) > 15:
                        raise EmuError("too many LDS instructions outstanding")
            elif op == "ds_read_b32":
                if self.lds is None:
                    raise EmuError("LDS access in a kernel without LDS")
                srcp, _, mods = a[1].partition(" ")
                off = 0
                if mods:
                    key, _, num = mods.partition(":")
                    if key != "offset":
                        raise EmuError(f"LDS modifier not emulated: {mods}")
                    off = int(num)
                addr = self.src_vec(srcp).astype(np.int64) + off
                if (addr % 4).any() or (addr < 0).any() or (addr + 4 > self.lds.size * 4).any():
                    raise EmuError("ds_read_b32 outside the LDS or misaligned")
                w = addr // 4
                if self.lds_pend is not None and self.lds_pend[w].any():
                    raise EmuError("LDS read of words an LDS DMA has not finished writing")
                dst = self.vreg(a[0], write=True)
                self.v[dst] = self.lds[w]
                self.lgkm.append([dst])
                if len(self.lgkm) > 15:
                    raise EmuError("too many LDS instructions outstanding")
            elif op in ("ds_read2_b32", "ds_read2st64_b32"):
                # two dwords per lane at base + u*offset0 and base + u*offset1 (8-bit offsets;
                # u = 4 bytes, or 256 bytes for st64) into an even-aligned register pair
                unit = 4 if op == "ds_read2_b32" else 256
                if self.lds is None:
                    raise EmuError("LDS access in a kernel without LDS")
                srcp, _, mods = a[1].partition(" ")
                offs = {}
                for mod in mods.split():
                    key, _, num = mod.partition(":")
                    if key not in ("offset0", "offset1") or not 0 <= int(num) <= 255:
                        raise EmuError(f"LDS modifier not emulated: {mod}")
                    offs[key] = int(num)
                base = self.src_vec(srcp).astype(np.int64)
                dst = self.vtuple(a[0], 2)
                for j, key in enumerate(("offset0", "offset1")):
                    addr = base + unit * offs.get(key, 0)
                    if (addr % 4).any() or (addr < 0).any() or (addr + 4 > self.lds.size * 4).any():
                        raise EmuError(f"{op} outside the LDS or misaligned")
                    w = addr // 4
                    if self.lds_pend is not None and self.lds_pend[w].any():
                        raise EmuError("LDS read of words an LDS DMA has not finished writing")
                    self.v[dst[j]] = self.lds[w]
                self.lgkm.append(list(dst))
                if len(self.lgkm) > 15:
                    raise EmuError("too many LDS instructions outstanding")
            elif op == "ds_bpermute_b32":
                # lane l receives data[((addr[l] + offset) >> 2) & 63] through the LDS crossbar
                srcp, _, mods = a[2].partition(" ")
                off = 0
                if mods:
                    key, _, num = mods.partition(":")
                    if key != "offset":
                        raise EmuError(f"ds_bpermute modifier not emulated: {mods}")
                    off = int(num)
                addr = self.src_vec(a[1]).astype(np.int64)
                data = self.v[self.vreg(srcp)].copy()
                dst = self.vreg(a[0], write=True)
                self.v[dst] = data[((addr + off) >> 2) & 63]
                self.lgkm.append([dst])
                if len(self.lgkm) > 15:
                    raise EmuError("too many LDS instructions outstanding")
            elif op == "v_add_f32_e32":
                x = self.src_vec(a[1]).view(np.float32)
                y = self.src_vec(a[2]).view(np.float32)
                self.wv(a[0], (x + y).view(np.uint32))
            elif op == "s_nop":
                self.valu += int(a[0]) + 1
            elif op == "s_mov_b32" and a[0] == "m0":
                self.m0, self.m0_wr = self.sval(a[1]), steps
            elif op == "s_add_u32" and a[0] == "m0":
                self.m0, self.m0_wr = (self.sval(a[1]) + self.sval(a[2])) & 0xFFFFFFFF, steps
            elif op == "s_mov_b32":
                self.s[self.sreg(a[0])] = self.sval(a[1])
            elif op in ("s_and_b32", "s_mul_i32", "s_lshr_b32", "s_add_u32", "s_sub_u32"):
                x, y = self.sval(a[1]), self.sval(a[2])
                r = {"s_and_b32": x & y, "s_mul_i32": x * y, "s_lshr_b32": x >> (y & 31),
                     "s_add_u32": x + y, "s_sub_u32": x - y}[op]
                if op == "s_add_u32":
                    self.scc = r > 0xFFFFFFFF
                self.s[self.sreg(a[0])] = r & 0xFFFFFFFF
            elif op == "s_cmp_lt_u32":
                self.scc = self.sval(a[0]) < self.sval(a[1])
            elif op == "s_cmp_eq_u32":
                self.scc = self.sval(a[0]) == self.sval(a[1])
            elif op == "s_cbranch_scc1":
                if self.scc:
                    pc = self.k.labels[a[0]]
            elif op == "s_cbranch_scc0":
                if not self.scc:
                    pc = self.k.labels[a[0]]
            elif op == "s_getpc_b64":
                m = _RANGE.match(a[0])
                self.s[int(m.group(2))] = pc
                self.s[int(m.group(3))] = 0
            elif op == "s_addc_u32":
                r = self.sval(a[1]) + self.sval(a[2]) + (1 if self.scc else 0)
                self.s[self.sreg(a[0])] = r & 0xFFFFFFFF
            elif op == "s_setpc_b64":
                m = _RANGE.match(a[0])
                pc = int(self.s[int(m.group(2))])
            elif op == "v_readfirstlane_b32":
                src = self.vreg(a[1])
                self.need(self.wr[src], 1, f"v_readfirstlane of v{src}")
                self.s[self.sreg(a[0])] = int(self.v[src][0])
                self.valu += 1
            elif op in ("v_lshrrev_b32_e32", "v_lshlrev_b32_e32", "v_and_b32_e32", "v_add_u32_e32",
                        "v_sub_u32_e32"):
                x = self.src_vec(a[1]).astype(np.uint64)
                y = self.src_vec(a[2]).astype(np.uint64)
                if op == "v_lshrrev_b32_e32":
                    r = y >> (x & 31)
                elif op == "v_lshlrev_b32_e32":
                    r = y << (x & 31)
                elif op == "v_and_b32_e32":
                    r = x & y
                elif op == "v_add_u32_e32":
                    r = x + y
                else:
                    r = x - y
                self.wv(a[0], (r & 0xFFFFFFFF).astype(np.uint32))
            elif op == "v_mov_b32_e32":
                self.wv(a[0], self.src_vec(a[1]))
            elif op == "v_bfrev_b32_e32":
                x = self.sval(a[1])
                self.wv(a[0], np.full(64, int(f"{x:032b}"[::-1], 2), np.uint32))
            elif op in ("v_mul_hi_u32", "v_mul_lo_u32"):
                x = self.src_vec(a[1]).astype(np.uint64)
                y = self.src_vec(a[2]).astype(np.uint64)
                p = x * y
                self.wv(a[0], ((p >> 32) if op == "v_mul_hi_u32" else p) & 0xFFFFFFFF)
            elif op == "v_cmp_gt_u32_e32":
                if a[0] != "vcc":
                    raise EmuError("v_cmp writes vcc only")
                self.vcc = self.src_vec(a[1]) > self.src_vec(a[2])
                self.vcc_wr = self.valu
                self.valu += 1
            elif op == "v_cndmask_b32_e32":
                if a[3] != "vcc":
                    raise EmuError("v_cndmask reads vcc only")
                self.need(self.vcc_wr, 2, "v_cndmask read of vcc")
                self.wv(a[0], np.where(self.vcc, self.src_vec(a[2]), self.src_vec(a[1])))
            elif op == "v_mov_b32_dpp":
                srcp, _, mods = a[1].partition(" ")
                if mods != "wave_shl:1 row_mask:0xf bank_mask:0xf":
                    raise EmuError(f"DPP control not emulated: {mods}")
                dst = self.vreg(a[0], write=True)
                src = self.vreg(srcp)
                self.need(self.wr[src], 2, f"DPP read of v{src}")
                out = self.v[dst].copy()
                out[:63] = self.v[src][1:]
                self.v[dst] = out
                self.wr[dst] = self.valu
                self.valu += 1
            elif op == "v_fmamk_f32":
                x = self.src_vec(a[1]).view(np.float32).astype(np.float64)
                k = np.float64(np.uint32(int(a[2], 0)).view(np.float32))
                z = self.src_vec(a[3]).view(np.float32).astype(np.float64)
                self.wv(a[0], (x * k + z).astype(np.float32).view(np.uint32))
            elif op == "v_fmac_f32_e32":
                k = self.src_vec(a[1]).view(np.float32).astype(np.float64)
                x = self.src_vec(a[2]).view(np.float32).astype(np.float64)
                d = self.v[self.vreg(a[0])].view(np.float32).astype(np.float64)
                self.wv(a[0], (k * x + d).astype(np.float32).view(np.uint32))
            elif op in ("buffer_load_dword", "buffer_load_dwordx4") and len(a) == 3:
                # LDS DMA: lane i writes its 1 (4) dwords at LDS byte m0 + 4*i (16*i); zero where
                # the offset is out of range
                so, _, mods = a[2].partition(" ")
                if mods != "offen lds":
                    raise EmuError(f"LDS DMA form not emulated: {mods}")
                if self.lds is None:
                    raise EmuError("LDS DMA in a kernel without LDS")
                if self.m0 is None or steps - self.m0_wr < 2:
                    raise EmuError("LDS DMA without a wait state after writing m0")
                lw = 4 if op == "buffer_load_dwordx4" else 1
                addr, nrec = self.rsrc(a[1])
                bi, arr = self.buffer(addr)
                voff = self.src_vec(a[0]).astype(np.uint64)
                soff = self.sval(so)
                off = voff + np.uint64(soff)
                inb = off < np.uint64(nrec)
                if ((voff < np.uint64(nrec)) != inb).any():
                    raise EmuError("range check would depend on the scalar offset")
                if (off[inb] % (4 * lw)).any():
                    raise EmuError("misaligned LDS DMA source")
                base = int(self.m0)
                if base % 4 or base < 0 or base + 64 * 4 * lw > self.lds.size * 4:
                    raise EmuError("LDS DMA outside the LDS")
                words = np.zeros(64 * lw, np.uint32)
                src_idx = (off[inb] // 4).astype(np.int64)
                if (src_idx + lw > arr.size).any():
                    raise EmuError("descriptor range larger than the buffer")
                lanes = np.nonzero(inb)[0]
                for j in range(lw):
                    words[lanes * lw + j] = arr[src_idx + j]
                dst = base // 4 + np.arange(64 * lw)
                self.lds[dst] = words
                self.lds_pend[dst] = True
                self._issue_vmem(("lds", dst))
            elif op == "buffer_load_dword" or op == "buffer_store_dword":
                so, _, mods = a[3].partition(" ")
                mods = mods.split()
                # stores may carry a cache policy (nt, sc0, sc1): it does not change the result
                if mods[:1] != ["offen"] or (op == "buffer_load_dword" and len(mods) > 1) or \
                        any(m not in ("nt", "sc0", "sc1") for m in mods[1:]):
                    raise EmuError("buffer access other than offen")
                addr, nrec = self.rsrc(a[2])
                bi, arr = self.buffer(addr)
                voff = self.src_vec(a[1]).astype(np.uint64)
                soff = self.sval(so)
                off = voff + np.uint64(soff)
                inb = off < np.uint64(nrec)
                if ((voff < np.uint64(nrec)) != inb).any():
                    raise EmuError("range check would depend on the scalar offset")
                if (off[inb] % 4).any():
                    raise EmuError("misaligned access")
                idx = (off[inb] // 4).astype(np.int64)
                if (idx >= arr.size).any():
                    raise EmuError("descriptor range larger than the buffer")
                if op == "buffer_load_dword":
                    d = self.vreg(a[0], write=True)
                    vals = np.zeros(64, np.uint32)
                    vals[inb] = arr[idx]
                    self.v[d] = vals
                    self.wr[d] = self.valu  # the DPP rule counts from the load's issue
                    self._issue_vmem(d)
                else:
                    d = self.vreg(a[0])
                    self.stores.append((bi, idx, self.v[d][inb].copy()))
                    self._issue_vmem(("store", None))
            else:
                raise EmuError(f"instruction not emulated: {op} {a}")


def run_baked(src: str, info: dict, x: np.ndarray, M: int, E: int, F: int):
    """Run a generated kernel over the batch x (N, C, H, W) and return y (N, M, E, F).

    ``info`` holds the handle's baked-plan fields (sparseconv_query): valid lanes, row
    pitch, groups and wavefronts per workgroup, from which the launch is set up exactly as
    the library's forward pass does."""
    k = Kernel(src)
    N = x.shape[0]
    V, Pb, G = info["bake_valid_lanes"], info["bake_pitch"], info["bake_groups"]
    Q, T = info["bake_splits"], info["bake_units_per_wg"]
    WPB = Q * T * (G if info.get("bake_shared_window") else 1)
    if info.get("bake_stage"):
        # staged kernels: positions of the padded layout (H + 2 pad rows of Pb words per image),
        # ntiles = workgroups of T tiles of 64 per group
        qtot = N * (info["H"] + 2 * info["pad"]) * Pb
        ntiles = (qtot + 64 * T - 1) // (64 * T)
        per_xcd = (ntiles * (1 if info.get("bake_sequential") or info.get("bake_shared_window") else G) + 7) // 8
    else:
        qtot = N * E * Pb
        ntiles = (qtot + V - 1) // V
        units = ntiles * G
        wgs = (units + T - 1) // T
        per_xcd = (wgs + 7) // 8
    xb = np.ascontiguousarray(x, np.float32).reshape(-1).view(np.uint32)
    y = np.full(N * M * E * F, 0x7FC00000, np.uint32)  # NaN: unwritten
    xaddr, yaddr = 0x10000000, 0x7F0000000
    kernarg = struct.pack("<QQIIIIII", xaddr, yaddr, N, ntiles, xb.size * 4, y.size * 4, qtot, per_xcd)
    written = np.zeros(y.size, np.int32)
    for b in range(8 * per_xcd):
        lds = np.full(max(k.lds_bytes, 4) // 4, 0x7FC00000, np.uint32) if k.lds_bytes else None
        pend = np.zeros(lds.size, bool) if lds is not None else None
        waves = [Wave(k, kernarg, b, w, [(xaddr, xb), (yaddr, y)], lds, pend) for w in range(WPB)]
        # run every wave up to its next barrier (or its end), then release the barrier; a
        # barrier waits only for the waves that have not ended
        gens = [w.run() for w in waves]
        live = list(range(WPB))
        while live:
            at_barrier = []
            for i in live:
                try:
                    next(gens[i])
                    at_barrier.append(i)
                except StopIteration:
                    pass
            live = at_barrier
        if len(set(w.barriers for w in waves if w.barriers)) > 1:
            # a workgroup barrier counts arrivals, not code positions: waves that pass a
            # different number of them would synchronise with the wrong partner barrier (waves
            # that end before any barrier, e.g. units past the last tile, take no part)
            raise EmuError(f"workgroup {b}: waves passed different numbers of barriers "
                           f"{[w.barriers for w in waves]}")
        for wave in waves:
            for bi, idx, vals in wave.stores:
                assert bi == 1, "store into the input"
                y[idx] = vals
                written[idx] += 1
    if (written > 1).any():
        raise EmuError(f"{int((written > 1).sum())} output elements stored more than once")
    return y.view(np.float32).reshape(N, M, E, F), written.reshape(N, M, E, F)
